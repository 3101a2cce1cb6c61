"""The differentiable calls (vsa_attention, block_sparse_attn_varlen_attention):
under autograd they must give exactly the forward and backward entry points'
results (out, dq, dk, dv bitwise; gate gradients as the fp32 ones rounded to
the gates' dtype), and the gradients must match the fp64 oracle; without
autograd they are the plain forward."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_close, dev, host64
from workloads import make_inputs

pytestmark = pytest.mark.gpu
BF16, F32 = torch.bfloat16, torch.float32


def _vsa():
    import trainable_block_sparse_cube_amd as vsa
    return vsa


def _leaves(inp, dtype):
    return [dev(inp[n], dtype).requires_grad_() for n in ("q", "k", "v", "gc", "gf")]


@pytest.mark.parametrize("dtype", [BF16, F32], ids=["bf16", "f32"])
def test_vsa_attention_matches_entry_points_and_oracle(dtype):
    vsa = _vsa()
    B, nh, D, grid, K = 2, 2, 64, (8, 8, 12), 4
    inp = make_inputs(B, nh, D, grid, dtype="bf16" if dtype == BF16 else "f32", seed=77, with_dout=True)
    leaves = _leaves(inp, dtype)
    do = dev(inp["dout"], dtype)
    out, sel = vsa.vsa_attention(*leaves, grid, K)
    (out * do).sum().backward()
    torch.cuda.synchronize()

    plain = [t.detach() for t in leaves]
    out_ref, sel_ref, saved = vsa.vsa_forward(*plain, grid, K, save=True)
    g_ref = vsa.vsa_backward(*plain, do, sel_ref, saved, grid)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref) and torch.equal(sel, sel_ref)
    for t, g in zip(leaves[:3], g_ref[:3]):
        assert t.grad.dtype == dtype and torch.equal(t.grad, g)
    for t, g in zip(leaves[3:], g_ref[3:]):
        assert t.grad.dtype == dtype and torch.equal(t.grad, g.to(dtype))

    lists = oracle.lists_from_sel(sel.cpu().numpy())
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], inp["dout"], grid, lists)
    for t, name in zip(leaves[:3], ("dq", "dk", "dv")):
        assert_close(host64(t.grad), ref[name], dtype, f"autograd {name}")
    # gate gradients: the fp32 ones (held to the usual bar by the backward
    # tests) rounded once more to the gates' dtype, so half a unit in the
    # last place of that dtype (2^-9 relative for bf16) joins the bound
    for t, name in zip(leaves[3:], ("dgc", "dgf")):
        g, r = host64(t.grad), ref[name]
        bound = (1e-4 if dtype == F32 else 2e-2) + (2.0 ** -9 if dtype == BF16 else 0.0) * np.abs(r)
        assert np.all(np.abs(g - r) <= bound), f"autograd {name}: {np.max(np.abs(g - r) - bound):.3e} over"


def test_vsa_attention_without_autograd_is_the_plain_forward():
    vsa = _vsa()
    B, nh, D, grid, K = 1, 2, 128, (8, 8, 8), 3
    inp = make_inputs(B, nh, D, grid, dtype="bf16", seed=78)
    q, k, v, gc, gf = (dev(inp[n], BF16) for n in ("q", "k", "v", "gc", "gf"))
    out, sel = vsa.vsa_attention(q, k, v, gc, gf, grid, K)
    ref, sel_ref, _ = vsa.vsa_forward(q, k, v, gc, gf, grid, K)
    assert not out.requires_grad and torch.equal(out, ref) and torch.equal(sel, sel_ref)
    leaves = _leaves(inp, BF16)
    with torch.no_grad():
        out2, _ = vsa.vsa_attention(*leaves, grid, K)
    assert not out2.requires_grad and torch.equal(out2, ref)


def test_varlen_attention_matches_entry_points():
    vsa = _vsa()
    B, nh, D, grid = 1, 2, 128, (8, 12, 16)
    nc = grid[0] * grid[1] * grid[2] // 64
    inp = make_inputs(B, nh, D, grid, dtype="bf16", seed=79, with_dout=True)
    rng = np.random.default_rng(80)
    lens = rng.integers(0, nc + 1, size=B * nh * nc)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ids = np.concatenate([np.sort(rng.choice(nc, int(n), replace=False)) for n in lens]).astype(np.int32)
    offs_d, ids_d = torch.from_numpy(offs).cuda(), torch.from_numpy(ids).cuda()
    leaves = _leaves(inp, BF16)
    do = dev(inp["dout"], BF16)
    out = vsa.block_sparse_attn_varlen_attention(*leaves, grid, offs_d, ids_d)
    (out * do).sum().backward()
    torch.cuda.synchronize()

    plain = [t.detach() for t in leaves]
    out_ref, saved = vsa.block_sparse_attn_varlen(*plain, grid, offs_d, ids_d, save=True)
    g_ref = vsa.block_sparse_attn_varlen_backward(*plain, do, offs_d, ids_d, saved, grid)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref)
    for t, g in zip(leaves, g_ref):
        assert torch.equal(t.grad, g.to(BF16))
