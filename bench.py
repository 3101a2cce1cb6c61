"""Benchmark of the VSA forward hot path on one MI355X.

One step = one vsa_forward call (cube permute + pooling, coarse attention
with top-K, block-sparse fine attention with the gated combine) on the
61440-token workload: B=1, 12 heads, head_dim 128, grid 20x48x64, top-K 32,
bf16 inputs already resident in HBM.  value = effective TFLOP/s of the
whole forward, counting the sparse FLOPs the method needs (fine stage QK^T
and PV over the selected cubes plus the dense coarse stage).

The fine kernel is also timed on its own (HIP events on the stream it is
launched on) for the roofline entry; the fp64 CPU oracle is timed on a
bounded sample of the same workload as the CPU baseline.
Prints one JSON line.
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="long61k")
    p.add_argument("--topk", type=int, default=32)
    p.add_argument("--cpu-heads", type=int, default=4,
                   help="heads of the workload the CPU oracle runs (bounded sample)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run one plain 1 GiB device copy (for scaling profiler byte counters)")
    p.add_argument("--extra", action="store_true",
                   help="also time top-K 16, the 70400-token workload, varlen and backward")
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


def cpu_baseline(inp, w, topk, heads):
    import numpy as np
    import oracle
    from workloads import coarse_flops, fine_flops
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = 1
    sl = slice(0, heads)
    args = [np.ascontiguousarray(inp[n][:, :, sl]) for n in ("q", "k", "v", "gc", "gf")]
    t0 = time.perf_counter()
    oracle.forward(*args, w.grid, topk)
    dt = time.perf_counter() - t0
    flops = fine_flops(w.B, heads, w.N, topk, w.head_dim) + coarse_flops(w.B, heads, w.n_cubes, w.head_dim)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"full fp64 forward of heads 0..{heads - 1} of {w.heads} (B={w.B}, grid "
                      f"{'x'.join(map(str, w.grid))}, top-K {topk}) in {dt:.1f} s; heads are independent",
            "seconds": dt, "cpu": platform.processor() or platform.machine()}


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
    qp, kp, vt, qc, kc, vc = vsa.vsa_cube_permute_pool(q, k, v, w.grid)
    oc, lse, sel2 = vsa.vsa_coarse_topk(qc, kc, vc, K)
    ms_pp = timed(lambda: vsa.vsa_cube_permute_pool(q, k, v, w.grid), a.steps, a.warmup, stream)
    ms_coarse = timed(lambda: vsa.vsa_coarse_topk(qc, kc, vc, K), a.steps, a.warmup, stream)
    fout = torch.empty_like(q)
    ms_fine = timed(lambda: vsa.vsa_fine_forward(qp, kp, vt, oc, gc, gf, w.grid, sel2, topk=K, out=fout),
                    a.steps, a.warmup, stream)

    f_fine = fine_flops(w.B, w.heads, w.N, K, w.head_dim)
    f_coarse = coarse_flops(w.B, w.heads, w.n_cubes, w.head_dim)
    elt = 2
    pp_bytes = 6 * w.B * w.N * w.heads * w.head_dim * elt + 3 * w.B * w.heads * w.n_cubes * w.head_dim * 4
    fine_tflops = f_fine / (ms_fine * 1e-3) / 1e12
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
        "stages_ms": {"permute_pool": ms_pp, "coarse_topk": ms_coarse, "fine": ms_fine},
        "permute_pool_GBs": pp_bytes / (ms_pp * 1e-3) / 1e9,
        "roofline": {"bound": "mfma", "kernel": "fine_fwd_bf16_kernel<128>",
                     "achieved": fine_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": fine_tflops / PEAK_BF16_TFLOPS, "traffic": None,
                     "flops_per_launch": f_fine},
    }
    if a.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = 1 << 30
    if a.extra:
        res["extra"] = extra(a, vsa, torch, w, stream)
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, w, K, min(a.cpu_heads, w.heads))
    print(json.dumps(res), flush=True)


def extra(a, vsa, torch, w, stream):
    from workloads import WORKLOADS, coarse_flops, fine_flops, fine_flops_lists, workload_inputs
    ext = {}
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda().contiguous()
    return ext


if __name__ == "__main__":
    main()
