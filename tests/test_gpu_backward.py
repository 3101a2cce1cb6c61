"""GPU parity of the backward (C ABI via the thin binding) against the fp64
oracle: full tensors at small sizes (bf16 and fp32) and at the training
workload size, sampled cubes at the largest accepted cube count,
determinism, and the argument checks of the backward entry points."""
import numpy as np
import pytest
import torch

import oracle
from oracle import vsa_oracle as vo
from tests.gpu_util import Stats, assert_close, dev, host64, log, per_head, sum_stats
from workloads import WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16
GRADS = ("dq", "dk", "dv", "dgc", "dgf")


def _vsa():
    import trainable_block_sparse_cube_amd as vsa
    return vsa


F32 = torch.float32


def _run(inp, grid, K, dtype=BF16):
    vsa = _vsa()
    q, k, v, gc, gf, do = (dev(inp[n], dtype) for n in ("q", "k", "v", "gc", "gf", "dout"))
    out, sel, saved = vsa.vsa_forward(q, k, v, gc, gf, grid, K, save=True)
    grads = vsa.vsa_backward(q, k, v, gc, gf, do, sel, saved, grid)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), grads


SMALL = [
    # B, heads, D, grid, topk
    (2, 2, 128, (8, 8, 12), 3),
    (1, 3, 64, (8, 12, 16), 5),
    (1, 2, 128, (8, 8, 8), 8),   # K = Nc: dense fine stage
    (2, 1, 128, (4, 4, 4), 1),   # a single cube
]


def _seeded_shapes(n, seed):
    """n small backward cases drawn once from a fixed seed: grid sides are
    multiples of 4 (1 to 3 cubes per side), 1-2 batches, 1-3 heads, D in
    {64, 128}, K from 1 to all cubes."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        grid = tuple(4 * int(x) for x in rng.integers(1, 4, size=3))
        nc = grid[0] * grid[1] * grid[2] // 64
        out.append((int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.choice([64, 128])), grid,
                    int(rng.integers(1, nc + 1))))
    return out


@pytest.mark.parametrize("case", SMALL + _seeded_shapes(6, 4048),
                         ids=lambda c: f"B{c[0]}h{c[1]}D{c[2]}g{'x'.join(map(str, c[3]))}k{c[4]}")
def test_backward_small_full_compare(case):
    B, nh, D, grid, K = case
    log(f"backward small {case}")
    inp = make_inputs(B, nh, D, grid, dtype="bf16", seed=200 + K, with_dout=True)
    sel, grads = _run(inp, grid, K)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], inp["dout"], grid,
                          oracle.lists_from_sel(sel))
    for name, g in zip(GRADS, grads):
        assert_close(host64(g), ref[name], BF16, name)


def test_backward_is_deterministic():
    grid = (8, 8, 16)
    inp = make_inputs(1, 2, 128, grid, dtype="bf16", seed=5, with_dout=True)
    _, g1 = _run(inp, grid, 4)
    _, g2 = _run(inp, grid, 4)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
def test_backward_takes_k_and_v_from_the_saved_state(dtype):
    """K and V enter the backward only through the tiles and cube means the
    forward left in its saved state: other k and v tensors handed to the
    backward change nothing."""
    vsa = _vsa()
    grid = (8, 8, 16)
    inp = make_inputs(1, 2, 64, grid, dtype="bf16" if dtype == BF16 else "f32", seed=77, with_dout=True)
    q, k, v, gc, gf, do = (dev(inp[n], dtype) for n in ("q", "k", "v", "gc", "gf", "dout"))
    out, sel, saved = vsa.vsa_forward(q, k, v, gc, gf, grid, 4, save=True)
    g1 = vsa.vsa_backward(q, k, v, gc, gf, do, sel, saved, grid)
    g2 = vsa.vsa_backward(q, torch.randn_like(k), torch.zeros_like(v), gc, gf, do, sel, saved, grid)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_varlen_backward_small_including_empty_lists():
    vsa = _vsa()
    B, nh, D, grid = 1, 2, 128, (8, 8, 12)
    log("varlen backward small")
    inp = make_inputs(B, nh, D, grid, dtype="bf16", seed=31, with_dout=True, varlen=(0, 12))
    offs = torch.from_numpy(inp["kv_offsets"]).cuda()
    ids = torch.from_numpy(inp["kv_ids"]).cuda()
    assert (np.diff(inp["kv_offsets"]) == 0).any()
    q, k, v, gc, gf, do = (dev(inp[n], BF16) for n in ("q", "k", "v", "gc", "gf", "dout"))
    out, saved = vsa.block_sparse_attn_varlen(q, k, v, gc, gf, grid, offs, ids, save=True)
    grads = vsa.block_sparse_attn_varlen_backward(q, k, v, gc, gf, do, offs, ids, saved, grid)
    torch.cuda.synchronize()
    lists = oracle.lists_from_csr(inp["kv_offsets"], inp["kv_ids"], B, nh, 12)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], inp["dout"], grid, lists)
    for name, g in zip(GRADS, grads):
        assert_close(host64(g), ref[name], BF16, name)


def test_varlen_backward_with_shuffled_lists():
    """The order inside a key list is free: with every list shuffled, dK, dV
    and the gate gradients (accumulated over the transposed lists, in query
    cube order) come out bitwise the same, and dQ (accumulated in list
    order, from the dS tile stored for each list entry) still matches the
    oracle.  Pins the entry-to-tile mapping of the dQ pass."""
    vsa = _vsa()
    B, nh, D, grid = 2, 2, 128, (8, 12, 16)  # 24 cubes
    inp = make_inputs(B, nh, D, grid, dtype="bf16", seed=37, with_dout=True, varlen=(1, 24))
    offs_np, ids_np = inp["kv_offsets"], inp["kv_ids"]
    rng = np.random.default_rng(38)
    shuffled = ids_np.copy()
    for a, b in zip(offs_np[:-1], offs_np[1:]):
        shuffled[a:b] = rng.permutation(shuffled[a:b])
    assert not np.array_equal(shuffled, ids_np)
    offs = torch.from_numpy(offs_np).cuda()
    q, k, v, gc, gf, do = (dev(inp[n], BF16) for n in ("q", "k", "v", "gc", "gf", "dout"))
    # one forward state for both (the forward's own rounding follows list order)
    _, saved = vsa.block_sparse_attn_varlen(q, k, v, gc, gf, grid, offs, torch.from_numpy(ids_np).cuda(),
                                            save=True)
    runs = []
    for ids_host in (ids_np, shuffled):
        ids = torch.from_numpy(ids_host).cuda()
        runs.append(vsa.block_sparse_attn_varlen_backward(q, k, v, gc, gf, do, offs, ids, saved, grid))
    torch.cuda.synchronize()
    for i, name in enumerate(GRADS):
        if name != "dq":
            assert torch.equal(runs[0][i], runs[1][i]), name
    lists = oracle.lists_from_csr(offs_np, ids_np, B, nh, 24)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], inp["dout"], grid, lists)
    assert_close(host64(runs[1][0]), ref["dq"], BF16, "dq, shuffled lists")


def test_backward_training_workload_whole_tensor():
    """train16k: B=2, 12 heads, head_dim 128, 16x32x32 grid, top-K 32.
    All five gradients over the whole tensors against oracle.backward under
    the GPU's selection (one (batch, head) per worker thread)."""
    w = WORKLOADS["train16k"]
    log("backward train16k: drawing inputs")
    inp = workload_inputs(w)
    sel, grads = _run(inp, w.grid, 32)
    g = [t.float().cpu().numpy() for t in grads]
    del grads

    def work(b, h):
        sl = lambda n: inp[n][b:b + 1, :, h:h + 1]
        ref = oracle.backward(sl("q"), sl("k"), sl("v"), sl("gc"), sl("gf"), sl("dout"), w.grid,
                              [[list(sel[b, h])]])
        return [Stats.of(g[0][b, :, h], ref["dq"][0, :, 0]), Stats.of(g[1][b, :, h], ref["dk"][0, :, 0]),
                Stats.of(g[2][b, :, h], ref["dv"][0, :, 0]), Stats.of(g[3][b, :, h], ref["dgc"][0, :, 0]),
                Stats.of(g[4][b, :, h], ref["dgf"][0, :, 0])]
    log(f"backward train16k: oracle on {w.B * w.heads} heads")
    res = per_head(work, [(b, h) for b in range(w.B) for h in range(w.heads)])
    for i, name in enumerate(GRADS):
        log("  " + sum_stats(r[i] for r in res).check(BF16, f"train16k {name}"))


def test_backward_at_the_largest_cube_count():
    """3584 cubes per (batch, head) (grid 4x32x1792, head_dim 64, one head),
    the most the library accepts: the list transpose at its largest LDS
    footprint, coarse GEMMs on 3584 x 3584 logits, long key lists for the
    dK/dV kernel.  Gradients of sampled query and key cubes against
    oracle.backward_sampled."""
    grid, K = (4, 32, 1792), 32
    log("backward at 3584 cubes: drawing inputs")
    inp = make_inputs(1, 1, 64, grid, dtype="bf16", seed=93, with_dout=True)
    sel, grads = _run(inp, grid, K)
    g = [t.float().cpu().numpy() for t in grads]
    for t in g:
        assert np.all(np.isfinite(t))
    members = vo.cube_members(*grid)
    rng = np.random.default_rng(6)
    qcs = [int(x) for x in rng.choice(3584, 4, replace=False)]
    kcs = [int(x) for x in rng.choice(3584, 4, replace=False)]
    out = oracle.backward_sampled(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], inp["dout"],
                                  grid, list(sel[0, 0]), 0, 0, qcs, kcs)
    acts = {n: [] for n in GRADS}
    refs = {n: [] for n in GRADS}
    for c in qcs:
        rows = members[c]
        acts["dq"].append(g[0][0, rows, 0]); refs["dq"].append(out[("dq", c)])
        acts["dgc"].append(g[3][0, rows, 0]); refs["dgc"].append(out[("dgc", c)])
        acts["dgf"].append(g[4][0, rows, 0]); refs["dgf"].append(out[("dgf", c)])
    for j in kcs:
        rows = members[j]
        acts["dk"].append(g[1][0, rows, 0]); refs["dk"].append(out[("dk", j)])
        acts["dv"].append(g[2][0, rows, 0]); refs["dv"].append(out[("dv", j)])
    for n in GRADS:
        assert_close(np.stack(acts[n]), np.stack(refs[n]), BF16, f"3584 cubes {n}")
    log("  3584 cubes: sampled gradients ok")


F32_CASES = [
    # B, heads, D, grid, topk
    (1, 2, 128, (8, 8, 12), 4),
    (2, 2, 64, (4, 8, 12), 3),
    (1, 3, 64, (8, 12, 16), 24),  # K = Nc: dense fine stage
    (2, 1, 128, (4, 4, 4), 1),    # a single cube
]


def test_backward_f32_tiny_workload():
    """The tiny fp32 workload (B=1, 2 heads, head_dim 64, 8x8x8, top-K 2)
    with dO ~ N(0, 1): all five gradients against the oracle at the fp32
    bar (max abs 1e-4)."""
    w = WORKLOADS["tiny_f32"]
    inp = make_inputs(w.B, w.heads, w.head_dim, w.grid, dtype="f32", seed=w.seed, with_dout=True)
    sel, grads = _run(inp, w.grid, w.topk[0], F32)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], inp["dout"], w.grid,
                          oracle.lists_from_sel(sel))
    for name, g in zip(GRADS, grads):
        assert g.dtype == F32
        m, _ = assert_close(host64(g), ref[name], F32, name)
        log(f"  tiny_f32 {name}: max abs {m:.2e}")


@pytest.mark.parametrize("case", F32_CASES,
                         ids=lambda c: f"B{c[0]}h{c[1]}D{c[2]}g{'x'.join(map(str, c[3]))}k{c[4]}")
def test_backward_f32_small_full_compare(case):
    B, nh, D, grid, K = case
    log(f"fp32 backward small {case}")
    inp = make_inputs(B, nh, D, grid, dtype="f32", seed=300 + K, with_dout=True)
    sel, grads = _run(inp, grid, K, F32)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], inp["dout"], grid,
                          oracle.lists_from_sel(sel))
    for name, g in zip(GRADS, grads):
        assert_close(host64(g), ref[name], F32, name)


def test_backward_f32_varlen_including_empty_lists():
    vsa = _vsa()
    B, nh, D, grid = 2, 2, 64, (8, 8, 12)
    inp = make_inputs(B, nh, D, grid, dtype="f32", seed=33, with_dout=True, varlen=(0, 12))
    assert (np.diff(inp["kv_offsets"]) == 0).any()
    offs = torch.from_numpy(inp["kv_offsets"]).cuda()
    ids = torch.from_numpy(inp["kv_ids"]).cuda()
    q, k, v, gc, gf, do = (dev(inp[n], F32) for n in ("q", "k", "v", "gc", "gf", "dout"))
    _, saved = vsa.block_sparse_attn_varlen(q, k, v, gc, gf, grid, offs, ids, save=True)
    grads = vsa.block_sparse_attn_varlen_backward(q, k, v, gc, gf, do, offs, ids, saved, grid)
    torch.cuda.synchronize()
    lists = oracle.lists_from_csr(inp["kv_offsets"], inp["kv_ids"], B, nh, 12)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], inp["dout"], grid, lists)
    for name, g in zip(GRADS, grads):
        assert_close(host64(g), ref[name], F32, name)


def test_backward_f32_is_deterministic():
    grid = (8, 8, 8)
    inp = make_inputs(1, 2, 128, grid, dtype="f32", seed=6, with_dout=True)
    _, g1 = _run(inp, grid, 3, F32)
    _, g2 = _run(inp, grid, 3, F32)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_backward_rejects_missing_state():
    vsa = _vsa()
    grid = (4, 4, 8)
    inp = make_inputs(1, 1, 64, grid, dtype="f32", seed=1, with_dout=True)
    q, k, v, gc, gf, do = (dev(inp[n], F32) for n in ("q", "k", "v", "gc", "gf", "dout"))
    out, sel, saved = vsa.vsa_forward(q, k, v, gc, gf, grid, 1, save=False)
    assert saved is None
    with pytest.raises(ValueError):
        vsa.vsa_backward(q, k, v, gc, gf, do, sel, saved, grid)
