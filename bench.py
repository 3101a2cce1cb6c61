"""Benchmark of the VSA forward hot path on one MI355X.

One step = one vsa_forward call (cube permute + pooling, coarse attention
with top-K, block-sparse fine attention with the gated combine) on the
61440-token workload: B=1, 12 heads, head_dim 128, grid 20x48x64, top-K 32,
bf16 inputs already resident in HBM.  value = effective TFLOP/s of the
whole forward, counting the sparse FLOPs the method needs (fine stage QK^T
and PV over the selected cubes plus the dense coarse stage).

The fine kernel is also timed on its own (HIP events on the stream it is
launched on, in the sorted processing order the forward gives it, and in
natural order for comparison) for the roofline entry, next to its compute
ceiling on the same data: the fine kernel on a shared selection (every query
cube picks the same key cubes, so every tile is an L2 hit).  The same line
carries the coarse stage's share of the step, the same shape with smooth
(video-like) cube means, whose neighbouring query cubes select overlapping
key cubes, the backward of the training
workload (B=2, 12 heads, 16x32x32, top-K 32) after its forward, and a dense
reference: the fine kernel with every key cube selected, whose MFU the
sparse fine stage is compared with.
The fp64 CPU oracle is timed on a bounded sample of the same workload as the
CPU baseline.  HBM traffic of the
fine kernel comes from the committed profiler-counter summary
(profiles/fine_fwd_bf16_long61k_k32_pmc.txt), as does its shader clock under
load (with the peak scaled to that clock beside the published one); both are
reported only while the kernel source still hashes to the value recorded
there.  Median and minimum per call come from a second pass with one event
pair per call.
Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
FINE_SRC = os.path.join(ROOT, "trainable_block_sparse_cube_amd", "csrc", "fine_fwd.hip")
DEVICE_H = os.path.join(ROOT, "trainable_block_sparse_cube_amd", "csrc", "vsa_device.h")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "fine_fwd_bf16_long61k_k32_pmc.txt")


def fine_source_hash():
    """Hash of what the bf16 fine kernel is built from: fine_fwd.hip without
    the fp32 kernel's function text, plus the device helper header."""
    src = open(FINE_SRC).read()
    head = "template <int D>\n__global__ __launch_bounds__(256) void fine_fwd_f32_kernel("
    i = src.index(head)
    j = src.index("\n}\n", i) + 3
    h = hashlib.sha256((src[:i] + src[j:]).encode())
    with open(DEVICE_H, "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def measured_counters():
    """The fine kernel's record in the committed counter summary (its last
    line is JSON: HBM bytes per launch, shader clock), or {} if absent or
    taken on other kernel source."""
    try:
        with open(PMC_SUMMARY) as f:
            rec = json.loads(f.read().strip().splitlines()[-1])
    except (OSError, ValueError, IndexError):
        return {}
    if rec.get("fine_fwd_source_sha256_16") != fine_source_hash():
        return {}
    return rec


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="long61k")
    p.add_argument("--topk", type=int, default=32)
    p.add_argument("--cpu-heads", type=int, default=8,
                   help="heads of the workload the CPU oracle runs (bounded sample)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run one plain 1 GiB device copy (for scaling profiler byte counters)")
    p.add_argument("--extra", action="store_true",
                   help="also time top-K 16, the 16K and 70400-token workloads, varlen, the mass rule "
                        "and smooth inputs")
    p.add_argument("--no-dense", action="store_true", help="skip the dense reference (about 0.1 s of GPU time)")
    p.add_argument("--no-backward", action="store_true", help="skip the training-workload backward")
    p.add_argument("--no-smooth", action="store_true", help="skip the smooth (video-like) selection case")
    return p.parse_args()


def timed(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def per_call_ms(fn, n, stream):
    """Median and minimum of n calls, each bracketed by its own events."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    fn()
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(n):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(n))
    return {"median": t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2]), "min": t[0], "calls": n}


def cpu_baseline(inp, w, topk, heads):
    import numpy as np
    import oracle
    from workloads import coarse_flops, fine_flops
    sl = slice(0, heads)
    args = [np.ascontiguousarray(inp[n][:, :, sl]) for n in ("q", "k", "v", "gc", "gf")]
    t0 = time.perf_counter()
    oracle.forward(*args, w.grid, topk)
    dt = time.perf_counter() - t0
    # thread pools as loaded by the run (the BLAS library loads on first use)
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        pools = [i for i in info if i.get("user_api") == "blas"] or info  # the oracle's numpy BLAS
        cores = max((i.get("num_threads", 1) for i in pools), default=1)
        blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in info
                                 if i.get("user_api") == "blas"})) or blas
    except Exception:  # pragma: no cover
        cores = 1
    cpu_model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    flops = fine_flops(w.B, heads, w.N, topk, w.head_dim) + coarse_flops(w.B, heads, w.n_cubes, w.head_dim)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"full fp64 forward of heads 0..{heads - 1} of {w.heads} (B={w.B}, grid "
                      f"{'x'.join(map(str, w.grid))}, top-K {topk}) in {dt:.1f} s; heads are independent",
            "seconds": dt, "cpu": cpu_model, "blas": blas}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the path shards over heads "
              "with no communication, so per-GPU throughput is the single-GPU figure.", file=sys.stderr)
        sys.exit(2)
    import torch
    import trainable_block_sparse_cube_amd as vsa
    from workloads import WORKLOADS, coarse_flops, fine_flops, workload_inputs

    w = WORKLOADS[a.workload]
    K = a.topk
    inp = workload_inputs(w, with_varlen=False)
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda().contiguous()
    q, k, v, gc, gf = (dev(inp[n]) for n in ("q", "k", "v", "gc", "gf"))
    stream = torch.cuda.current_stream()

    out, sel, _ = vsa.vsa_forward(q, k, v, gc, gf, w.grid, K)
    step = lambda: vsa.vsa_forward(q, k, v, gc, gf, w.grid, K)
    ms_step = timed(step, a.steps, a.warmup, stream)

    # stages on their own, same stream
    _, kp, vp, qc, kc, vc = vsa.vsa_cube_permute_pool(q, k, v, w.grid, with_q_tiles=False)
    oc, lse, sel2 = vsa.vsa_coarse_topk(qc, kc, vc, K, input_dtype=torch.bfloat16)
    ms_pp = timed(lambda: vsa.vsa_cube_permute_pool(q, k, v, w.grid, with_q_tiles=False),
                  a.steps, a.warmup, stream)
    ms_coarse = timed(lambda: vsa.vsa_coarse_topk(qc, kc, vc, K, input_dtype=torch.bfloat16), a.steps, a.warmup, stream)
    # the processing order the forward gives the fine kernel (query cubes
    # sorted by where their lists' quarter points lie), and the fine kernel with it
    order = vsa.vsa_fine_order(sel2, w.B, w.heads, w.n_cubes, topk=K)
    ms_order = timed(lambda: vsa.vsa_fine_order(sel2, w.B, w.heads, w.n_cubes, topk=K), a.steps, a.warmup, stream)
    fout = torch.empty_like(q)
    ms_fine = timed(lambda: vsa.vsa_fine_forward(q, kp, vp, oc, gc, gf, w.grid, sel2, topk=K, out=fout,
                                                 order=order), a.steps, a.warmup, stream)
    ms_fine_natural = timed(lambda: vsa.vsa_fine_forward(q, kp, vp, oc, gc, gf, w.grid, sel2, topk=K, out=fout),
                            a.steps, a.warmup, stream)

    f_fine = fine_flops(w.B, w.heads, w.N, K, w.head_dim)
    f_coarse = coarse_flops(w.B, w.heads, w.n_cubes, w.head_dim)
    elt = 2
    tok_bytes = w.B * w.N * w.heads * w.head_dim * elt          # one of q, k, v
    pooled_bytes = w.B * w.heads * w.n_cubes * w.head_dim * 4   # one fp32 mean tensor
    pp_bytes = 3 * tok_bytes + 2 * tok_bytes + 3 * pooled_bytes  # read q,k,v; write K, V tiles + means
    coarse_bytes = 4 * pooled_bytes + w.B * w.heads * w.n_cubes * (4 + 4 * K)
    fine_tflops = f_fine / (ms_fine * 1e-3) / 1e12

    # compute ceiling of the fine kernel on the same data
    tile_bytes = w.B * w.heads * w.n_cubes * K * 2 * 64 * w.head_dim * elt  # K and V tiles read
    shared = torch.arange(K, dtype=torch.int32, device="cuda").expand(w.B, w.heads, w.n_cubes, K).contiguous()
    ms_shared = timed(lambda: vsa.vsa_fine_forward(q, kp, vp, oc, gc, gf, w.grid, shared, topk=K, out=fout),
                      a.steps, a.warmup, stream)
    del shared
    calls = {"step": per_call_ms(step, a.steps, stream),
             "fine": per_call_ms(lambda: vsa.vsa_fine_forward(q, kp, vp, oc, gc, gf, w.grid, sel2, topk=K,
                                                             out=fout, order=order), a.steps, stream)}
    counters = measured_counters()
    clk = counters.get("fine_clock_GHz")
    res = {
        "metric": "VSA fwd effective TFLOP/s & % bf16 MFMA peak at 61440 tokens, K=32",
        "value": (f_fine + f_coarse) / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B}, heads={w.heads}, head_dim={w.head_dim}, "
                               f"grid {'x'.join(map(str, w.grid))} = {w.N} tokens, top-K {K}",
                   "B": w.B, "heads": w.heads, "head_dim": w.head_dim, "grid": list(w.grid),
                   "tokens": w.N, "topk": K, "parallelism": "single GPU"},
        "frac_of_peak_whole_forward": (f_fine + f_coarse) / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "stages_ms": {"permute_pool": ms_pp, "coarse_topk": ms_coarse, "fine_order": ms_order,
                      "fine": ms_fine, "fine_in_natural_order": ms_fine_natural},
        # the pages report the unfused coarse top-K at about 14 % of runtime
        "coarse_share_of_step": ms_coarse / ms_step,
        "stage_GBs": {"permute_pool": pp_bytes / (ms_pp * 1e-3) / 1e9,
                      "coarse_topk": coarse_bytes / (ms_coarse * 1e-3) / 1e9},
        "fine_TFLOPs": fine_tflops,
        "roofline": {"bound": "mfma", "kernel": "fine_fwd_bf16_kernel<128>",
                     "achieved": fine_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": fine_tflops / PEAK_BF16_TFLOPS, "traffic": counters.get("hbm_bytes_per_launch"),
                     "flops_per_launch": f_fine, "ms_per_launch": ms_fine,
                     # the kernel's own shader clock under load (profiler counters) and the
                     # peak and fraction at that clock; the published peak assumes 2.4 GHz
                     "clock_GHz": clk,
                     "peak_at_clock": PEAK_BF16_TFLOPS * clk / 2.4 if clk else None,
                     "frac_at_clock": fine_tflops / (PEAK_BF16_TFLOPS * clk / 2.4) if clk else None,
                     # MFMA utilisation from the counters: busy cycles over all SIMDs' cycles
                     "mfma_busy_frac_counters": counters.get("fine_mfma_busy_frac"),
                     # the measured HBM traffic (counters) over this launch time, against the
                     # 8 TB/s HBM peak: the tile re-reads that miss L2 are what bound the kernel
                     "traffic_TBps": (counters["hbm_bytes_per_launch"] / (ms_fine * 1e-3) / 1e12
                                      if counters.get("hbm_bytes_per_launch") else None),
                     "traffic_frac_of_hbm_peak": (counters["hbm_bytes_per_launch"] / (ms_fine * 1e-3) / 1e12
                                                  / (PEAK_HBM_GBS / 1000.0) if counters.get("hbm_bytes_per_launch") else None)},
        "per_call_ms": calls,
        "fine_floors": {
            "tile_bytes_per_launch": tile_bytes,
            "tile_delivery_TBps": tile_bytes / (ms_fine * 1e-3) / 1e12,
            "shared_selection_ms": ms_shared,
            "shared_selection_TFLOPs": f_fine / (ms_shared * 1e-3) / 1e12,
        },
    }
    del kp, vp, fout, q, k, v, gc, gf, out
    if not a.no_smooth:
        res["smooth_selections"] = smooth_case(vsa, torch, stream, a)
    if not a.no_backward:
        res["backward_train16k"] = backward_case(vsa, torch, stream, a)
    if not a.no_dense:
        res["dense_reference"] = dense_case(vsa, torch, stream, ms_step, fine_tflops,
                                            inp if w.name == "long61k" else None)
    if a.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = 1 << 30
    if a.extra:
        res["extra"] = extra(a, vsa, torch, stream)
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, w, K, min(a.cpu_heads, w.heads))
    print(json.dumps(res), flush=True)


def extra(a, vsa, torch, stream):
    """Other workloads, each timed the same way (HIP events, inputs resident)."""
    from workloads import WORKLOADS, coarse_flops, fine_flops, fine_flops_lists, workload_inputs
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda().contiguous()
    ext = {}
    steps, warm = max(3, a.steps // 2), 2

    def fwd_case(name, K):
        w = WORKLOADS[name]
        inp = workload_inputs(w, with_varlen=False)
        q, k, v, gc, gf = (dev(inp[n]) for n in ("q", "k", "v", "gc", "gf"))
        ms = timed(lambda: vsa.vsa_forward(q, k, v, gc, gf, w.grid, K), steps, warm, stream)
        fl = fine_flops(w.B, w.heads, w.N, K, w.head_dim) + coarse_flops(w.B, w.heads, w.n_cubes, w.head_dim)
        # the coarse stage's share of the forward at this length
        _, _, _, qc, kc, vc = vsa.vsa_cube_permute_pool(q, k, v, w.grid, with_q_tiles=False)
        ms_c = timed(lambda: vsa.vsa_coarse_topk(qc, kc, vc, K, input_dtype=torch.bfloat16), steps, warm, stream)
        return {"ms": ms, "TFLOPs": fl / (ms * 1e-3) / 1e12, "coarse_topk_ms": ms_c,
                "coarse_share": ms_c / ms}

    # the stand-in variable-length rule (mass 0.2 of the coarse probability,
    # lists clamped to [8, 64]) on the headline shape
    w = WORKLOADS["long61k"]
    inp = workload_inputs(w, with_varlen=False)
    q, k, v, gc, gf = (dev(inp[n]) for n in ("q", "k", "v", "gc", "gf"))
    _, offs, _, _ = vsa.vsa_forward_mass(q, k, v, gc, gf, w.grid, 0.2, 8, 64, trim=False)
    n_pairs = int(offs[-1].item())
    ms = timed(lambda: vsa.vsa_forward_mass(q, k, v, gc, gf, w.grid, 0.2, 8, 64, trim=False),
               steps, warm, stream)
    fl = fine_flops_lists(n_pairs, w.head_dim) + coarse_flops(w.B, w.heads, w.n_cubes, w.head_dim)
    ext["long61k_mass0.2_forward"] = {"ms": ms, "TFLOPs": fl / (ms * 1e-3) / 1e12,
                                      "mean_list_len": n_pairs / (w.B * w.heads * w.n_cubes),
                                      "rule": "shortest logit-ranked prefix with coarse mass >= 0.2, "
                                              "length clamped to [8, 64] (stand-in, not the pages' router)"}
    del q, k, v, gc, gf, offs, inp

    ext["long61k_k32_forward"] = fwd_case("long61k", 32)
    ext["long61k_k16_forward"] = fwd_case("long61k", 16)
    ext["pretrain16k_k32_forward"] = fwd_case("pretrain16k", 32)
    ext["large70k_k32_forward"] = fwd_case("large70k", 32)

    w = WORKLOADS["large70k"]
    inp = workload_inputs(w)
    q, k, v, gc, gf = (dev(inp[n]) for n in ("q", "k", "v", "gc", "gf"))
    offs = torch.from_numpy(inp["kv_offsets"]).cuda()
    ids = torch.from_numpy(inp["kv_ids"]).cuda()
    vsa.block_sparse_attn_varlen(q, k, v, gc, gf, w.grid, offs, ids)  # lists checked once
    ms = timed(lambda: vsa.block_sparse_attn_varlen(q, k, v, gc, gf, w.grid, offs, ids, validate=False),
               steps, warm, stream)
    fl = fine_flops_lists(int(ids.numel()), w.head_dim) + coarse_flops(w.B, w.heads, w.n_cubes, w.head_dim)
    ext["large70k_varlen_forward"] = {"ms": ms, "TFLOPs": fl / (ms * 1e-3) / 1e12,
                                      "mean_list_len": int(ids.numel()) / (w.B * w.heads * w.n_cubes)}
    del q, k, v, gc, gf, offs, ids, inp

    return ext


def smooth_case(vsa, torch, stream, a):
    """The headline shape with spatially smooth cube means: neighbouring
    query cubes select overlapping key cubes, as in video.  Context beside
    the random-selection headline, not the metric."""
    from workloads import WORKLOADS, coarse_flops, fine_flops, workload_inputs
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda().contiguous()
    steps, warm = max(3, a.steps // 2), 2
    w = WORKLOADS["long61k_smooth"]
    inp = workload_inputs(w, with_varlen=False)
    q, k, v, gc, gf = (dev(inp[n]) for n in ("q", "k", "v", "gc", "gf"))
    del inp
    _, kp, vp, qc, kc, vc = vsa.vsa_cube_permute_pool(q, k, v, w.grid, with_q_tiles=False)
    oc, _, sel = vsa.vsa_coarse_topk(qc, kc, vc, 32, input_dtype=torch.bfloat16)
    fout = torch.empty_like(q)
    order_s = vsa.vsa_fine_order(sel, w.B, w.heads, w.n_cubes, topk=32)
    ms_fine_s = timed(lambda: vsa.vsa_fine_forward(q, kp, vp, oc, gc, gf, w.grid, sel, topk=32, out=fout,
                                                   order=order_s), steps, warm, stream)
    ms_fwd_s = timed(lambda: vsa.vsa_forward(q, k, v, gc, gf, w.grid, 32), steps, warm, stream)
    s_np = sel[0, 0].cpu().numpy()
    f_s = fine_flops(w.B, w.heads, w.N, 32, w.head_dim)
    return {
        "workload": "long61k with smooth cube means (video-like selections), top-K 32",
        "forward_ms": ms_fwd_s,
        "forward_TFLOPs": (f_s + coarse_flops(w.B, w.heads, w.n_cubes, w.head_dim)) / (ms_fwd_s * 1e-3) / 1e12,
        "fine_ms": ms_fine_s, "fine_TFLOPs": f_s / (ms_fine_s * 1e-3) / 1e12,
        "fine_frac_of_peak": f_s / (ms_fine_s * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "mean_shared_ids_with_next_cube": float(sum(len(set(s_np[c]) & set(s_np[c + 1]))
                                                   for c in range(len(s_np) - 1)) / (len(s_np) - 1))}


def backward_case(vsa, torch, stream, a):
    """Forward with saved state, then the backward, on the training workload
    (B=2, 12 heads, head_dim 128, 16x32x32, top-K 32)."""
    from workloads import WORKLOADS, coarse_flops, fine_flops, workload_inputs
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda().contiguous()
    steps, warm = max(3, a.steps // 2), 3
    w = WORKLOADS["train16k"]
    inp = workload_inputs(w)
    q, k, v, gc, gf, do = (dev(inp[n]) for n in ("q", "k", "v", "gc", "gf", "dout"))
    out, sel, saved = vsa.vsa_forward(q, k, v, gc, gf, w.grid, 32, save=True)
    ms_f = timed(lambda: vsa.vsa_forward(q, k, v, gc, gf, w.grid, 32, save=True), steps, warm, stream)
    ms_b = timed(lambda: vsa.vsa_backward(q, k, v, gc, gf, do, sel, saved, w.grid), steps, warm, stream)
    ff = fine_flops(w.B, w.heads, w.N, 32, w.head_dim)
    fc = coarse_flops(w.B, w.heads, w.n_cubes, w.head_dim)
    tf_b = (2.5 * ff + 2 * fc) / (ms_b * 1e-3) / 1e12
    return {"workload": f"{w.name}: B={w.B}, heads={w.heads}, head_dim={w.head_dim}, "
                        f"grid {'x'.join(map(str, w.grid))}, top-K 32",
            "forward_ms": ms_f, "backward_ms": ms_b,
            "forward_TFLOPs": (ff + fc) / (ms_f * 1e-3) / 1e12,
            "backward_TFLOPs": tf_b, "backward_frac_of_peak": tf_b / PEAK_BF16_TFLOPS,
            "backward_flop_model": "2.5 x fine forward + 2 x coarse forward"}


def dense_case(vsa, torch, stream, ms_step, sparse_fine_tflops, inp=None):
    """Dense reference on the headline shape through the same fine kernel:
    every query cube lists all Nc key cubes (block attention over the whole
    clip).  Reports its MFU, the sparse fine stage's MFU as a share of it
    (the pages' figure of merit is 85 % of FlashAttention-3 MFU) and the
    whole VSA forward's speedup over dense fine attention.  Run last: its
    long launches heat the device.  `inp`: the headline's host inputs when
    the caller already drew them."""
    from workloads import WORKLOADS, fine_flops, workload_inputs
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda().contiguous()
    w = WORKLOADS["long61k"]
    if inp is None:
        inp = workload_inputs(w, with_varlen=False)
    q, k, v, gc, gf = (dev(inp[n]) for n in ("q", "k", "v", "gc", "gf"))
    _, kp, vp, qc, kc, vc = vsa.vsa_cube_permute_pool(q, k, v, w.grid, with_q_tiles=False)
    oc, _, _ = vsa.vsa_coarse_topk(qc, kc, vc, 0, input_dtype=torch.bfloat16)
    nc = w.n_cubes
    full = torch.arange(nc, dtype=torch.int32, device="cuda").expand(w.B, w.heads, nc, nc).contiguous()
    fout = torch.empty_like(q)
    ms_dense = timed(lambda: vsa.vsa_fine_forward(q, kp, vp, oc, gc, gf, w.grid, full, topk=nc, out=fout),
                     2, 1, stream)
    tf = fine_flops(w.B, w.heads, w.N, nc, w.head_dim) / (ms_dense * 1e-3) / 1e12
    return {"what": "fine kernel with K = Nc = 960 on the headline shape",
            "ms": ms_dense, "TFLOPs": tf, "frac_of_peak": tf / PEAK_BF16_TFLOPS,
            "sparse_fine_mfu_over_dense_mfu": sparse_fine_tflops / tf,
            "speedup_vsa_k32_forward_over_dense_fine": ms_dense / ms_step}


if __name__ == "__main__":
    main()
