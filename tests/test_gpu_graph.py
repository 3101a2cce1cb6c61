"""vsa_forward_noalloc under HIP graph capture, the use it exists for: the
forward is captured once (through torch's graph API, on its capture
stream) and replayed on fresh input values written into the same buffers,
with eager work and synchronizations between the replays; every replay must
equal an eager vsa_forward on those values bitwise (output and ids).  The
forward queues kernels only (no memsets, no host copies), so it records as
plain kernel nodes."""
import pytest
import torch

from tests.gpu_util import dev, log
from tests.test_zz_no_alloc import _noalloc
from workloads import make_inputs

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16


def test_noalloc_forward_replays_in_a_graph():
    import trainable_block_sparse_cube_amd as vsa
    from trainable_block_sparse_cube_amd import _lib
    lib = _lib.load()
    B, nh, D, grid, K = 1, 3, 128, (8, 12, 16), 5
    names = ("q", "k", "v", "gc", "gf")
    bufs = [dev(make_inputs(B, nh, D, grid, dtype="bf16", seed=300)[n], BF16) for n in names]
    out = torch.empty_like(bufs[0])
    sel = torch.empty((B, nh, 24, K), dtype=torch.int32, device="cuda")
    # first call outside the capture: it looks up the device's scratch array
    assert _noalloc(lib, *bufs, grid, K, out, sel, None) == _lib.VSA_OK
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = _noalloc(lib, *bufs, grid, K, out, sel, None)
    assert st == _lib.VSA_OK, lib.vsa_status_string(st)
    for r in range(4):
        log(f"graph replay {r}")
        fresh = make_inputs(B, nh, D, grid, dtype="bf16", seed=301 + r)
        for b, n in zip(bufs, names):
            b.copy_(dev(fresh[n], BF16))
        out.fill_(float("nan"))
        sel.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_out, ref_sel, _ = vsa.vsa_forward(*bufs, grid, K)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {r}: output"
        assert torch.equal(sel, ref_sel), f"replay {r}: ids"
