"""vsa_forward_noalloc (the forward for callers that cannot allocate, with
its workspace in the library's fixed device array) through the C ABI,
against vsa_forward on the same inputs: two calls in a row, the second on a
smaller input, outputs, ids and saved state bitwise equal; a shape whose
workspace exceeds the array is refused and leaves the output untouched."""
import ctypes

import numpy as np
import pytest
import torch

from tests.gpu_util import dev, log
from tests.test_gpu_forward import unpack_saved
from workloads import make_inputs

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16


def _noalloc(lib, q, k, v, gc, gf, grid, K, out, sel, saved):
    B, N, nh, D = q.shape
    dt = 1 if q.dtype == BF16 else 0
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    return lib.vsa_forward_noalloc(p(q), p(k), p(v), p(gc), p(gf), B, nh, D, *grid, K, dt, p(out), p(sel),
                                   p(saved), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_noalloc_forward_equals_vsa_forward_on_two_calls():
    import trainable_block_sparse_cube_amd as vsa
    from trainable_block_sparse_cube_amd import _lib
    lib = _lib.load()
    cases = [
        # the largest workload the fixed array holds: 12 heads x 16384 tokens, head_dim 128, K 32
        (1, 12, 128, (16, 32, 32), 32, BF16, 1001),
        # then a smaller one: the array keeps the first call's contents
        (1, 2, 64, (8, 8, 12), 3, BF16, 17),
        (1, 2, 64, (8, 8, 8), 2, torch.float32, 1000),
    ]
    for B, nh, D, grid, K, dt, seed in cases:
        log(f"noalloc forward B={B} heads={nh} D={D} grid={grid} K={K} {dt}")
        inp = make_inputs(B, nh, D, grid, dtype="bf16" if dt == BF16 else "f32", seed=seed)
        q, k, v, gc, gf = (dev(inp[n], dt) for n in ("q", "k", "v", "gc", "gf"))
        ref_out, ref_sel, ref_saved = vsa.vsa_forward(q, k, v, gc, gf, grid, K, save=True)
        out = torch.full_like(q, float("nan"))
        sel = torch.full_like(ref_sel, -1)
        saved = torch.zeros_like(ref_saved)
        st = _noalloc(lib, q, k, v, gc, gf, grid, K, out, sel, saved)
        torch.cuda.synchronize()
        assert st == _lib.VSA_OK, lib.vsa_status_string(st)
        assert torch.equal(out, ref_out)
        assert torch.equal(sel, ref_sel)
        # saved state field by field (the bytes between its aligned fields are never written)
        N = int(np.prod(grid))
        for a, b in zip(unpack_saved(saved, B, nh, N, D), unpack_saved(ref_saved, B, nh, N, D)):
            assert torch.equal(a, b)
        # inference form (no saved state)
        out2 = torch.full_like(q, float("nan"))
        assert _noalloc(lib, q, k, v, gc, gf, grid, K, out2, sel, None) == _lib.VSA_OK
        torch.cuda.synchronize()
        assert torch.equal(out2, ref_out)


def test_noalloc_forward_refuses_a_workspace_beyond_the_array():
    from trainable_block_sparse_cube_amd import _lib
    lib = _lib.load()
    B, nh, D, grid, K = 2, 12, 128, (16, 32, 32), 32  # about 215 MB of workspace
    assert lib.vsa_forward_workspace_bytes(B, nh, D, *grid, _lib.VSA_BF16) > (128 << 20)
    inp = make_inputs(B, nh, D, grid, dtype="bf16", seed=5)
    q, k, v, gc, gf = (dev(inp[n], BF16) for n in ("q", "k", "v", "gc", "gf"))
    out = torch.full_like(q, float("nan"))
    sel = torch.full((B, nh, np.prod(grid) // 64, K), -1, dtype=torch.int32, device="cuda")
    st = _noalloc(lib, q, k, v, gc, gf, grid, K, out, sel, None)
    torch.cuda.synchronize()
    assert st == _lib.VSA_ERR_WORKSPACE
    assert bool(torch.isnan(out.float()).all()) and bool((sel == -1).all())
