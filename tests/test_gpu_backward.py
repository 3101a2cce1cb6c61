"""GPU parity of the backward (C ABI via the thin binding) against the fp64
oracle: full tensors at small sizes, sampled cubes at the training workload
size, determinism, and the argument checks of the backward entry points."""
import numpy as np
import pytest
import torch

import oracle
from oracle import vsa_oracle as vo
from tests.gpu_util import assert_close, dev, host64, log
from workloads import WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16
GRADS = ("dq", "dk", "dv", "dgc", "dgf")


def _vsa():
    import trainable_block_sparse_cube_amd as vsa
    return vsa


def _run(inp, grid, K):
    vsa = _vsa()
    q, k, v, gc, gf, do = (dev(inp[n], BF16) for n in ("q", "k", "v", "gc", "gf", "dout"))
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


def test_backward_training_workload_sampled():
    """train16k: B=2, 12 heads, head_dim 128, 16x32x32 grid, top-K 32.
    Gradients of sampled query and key cubes against the fp64 oracle."""
    w = WORKLOADS["train16k"]
    log("backward train16k: drawing inputs")
    inp = workload_inputs(w)
    sel, grads = _run(inp, w.grid, 32)
    g = [t.float().cpu().numpy() for t in grads]
    for t in g:
        assert np.all(np.isfinite(t))
    members = vo.cube_members(*w.grid)
    rng = np.random.default_rng(4)
    acts = {n: [] for n in GRADS}
    refs = {n: [] for n in GRADS}
    for _ in range(4):
        b, h = int(rng.integers(w.B)), int(rng.integers(w.heads))
        qcs = [int(x) for x in rng.choice(w.n_cubes, 3, replace=False)]
        kcs = [int(x) for x in rng.choice(w.n_cubes, 3, replace=False)]
        out = oracle.backward_sampled(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], inp["dout"],
                                      w.grid, list(sel[b, h]), b, h, qcs, kcs)
        for c in qcs:
            rows = members[c]
            acts["dq"].append(g[0][b, rows, h]); refs["dq"].append(out[("dq", c)])
            acts["dgc"].append(g[3][b, rows, h]); refs["dgc"].append(out[("dgc", c)])
            acts["dgf"].append(g[4][b, rows, h]); refs["dgf"].append(out[("dgf", c)])
        for j in kcs:
            rows = members[j]
            acts["dk"].append(g[1][b, rows, h]); refs["dk"].append(out[("dk", j)])
            acts["dv"].append(g[2][b, rows, h]); refs["dv"].append(out[("dv", j)])
    for n in GRADS:
        assert_close(np.stack(acts[n]), np.stack(refs[n]), BF16, f"train16k {n}")
    log("  train16k sampled gradients ok")


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


def test_backward_rejects_fp32_and_missing_state():
    vsa = _vsa()
    from trainable_block_sparse_cube_amd import _lib
    grid = (4, 4, 8)
    inp = make_inputs(1, 1, 64, grid, dtype="f32", seed=1, with_dout=True)
    q, k, v, gc, gf, do = (dev(inp[n], torch.float32) for n in ("q", "k", "v", "gc", "gf", "dout"))
    out, sel, saved = vsa.vsa_forward(q, k, v, gc, gf, grid, 1, save=True)
    with pytest.raises(_lib.VSAError) as e:
        vsa.vsa_backward(q, k, v, gc, gf, do, sel, saved, grid)
    assert e.value.status == _lib.VSA_ERR_UNSUPPORTED
