"""The forward and backward at the largest (batch, head) count the library
accepts: B*heads = 65535 (a grid dimension of the coarse and permute
launches), here B = 5 and 13107 heads on a one-cube grid, top-K 1.  The
output and gradients start as NaN (an unwritten row cannot pass), every
value must come back finite, and sampled (batch, head) pairs, the first and
last among them, match the fp64 oracle.  The oracle runs only on the
sampled heads; each head is independent of the others."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import assert_close, dev, host64, log
from workloads import make_inputs

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16


def _vsa():
    import trainable_block_sparse_cube_amd as vsa
    return vsa


def test_forward_and_backward_at_the_largest_batch_head_count():
    vsa = _vsa()
    B, nh, D, grid, K = 5, 13107, 64, (4, 4, 4), 1
    assert B * nh == 65535
    log("65535 (batch, head) pairs: drawing inputs")
    inp = make_inputs(B, nh, D, grid, dtype="bf16", seed=211, with_dout=True)
    q, k, v, gc, gf, do = (dev(inp[n], BF16) for n in ("q", "k", "v", "gc", "gf", "dout"))
    out = torch.full_like(q, float("nan"))
    _, sel, saved = vsa.vsa_forward(q, k, v, gc, gf, grid, K, save=True, out=out)
    grads = vsa.vsa_backward(q, k, v, gc, gf, do, sel, saved, grid)
    torch.cuda.synchronize()
    del q, k, v, gc, gf, do, saved
    assert torch.equal(sel.cpu(), torch.zeros_like(sel.cpu()))  # one cube: it selects itself
    assert bool(torch.isfinite(out.float()).all())
    for name, g in zip(("dq", "dk", "dv", "dgc", "dgf"), grads):
        assert bool(torch.isfinite(g.float()).all()), name

    rng = np.random.default_rng(212)
    pairs = [(0, 0), (B - 1, nh - 1)] + [(int(b), int(h)) for b, h in
                                         zip(rng.integers(0, B, 10), rng.integers(0, nh, 10))]
    log(f"  checking {len(pairs)} sampled (batch, head) pairs against the oracle")
    for b, h in pairs:
        sl = lambda n: inp[n][b:b + 1, :, h:h + 1]
        lists = [[[0]]]
        ref = oracle.forward_with_sets(sl("q"), sl("k"), sl("v"), sl("gc"), sl("gf"), grid, lists)
        assert_close(host64(out[b:b + 1, :, h:h + 1]), ref["o"], BF16, f"out b{b} h{h}")
        g = oracle.backward(sl("q"), sl("k"), sl("v"), sl("gc"), sl("gf"), sl("dout"), grid, lists)
        for name, t in zip(("dq", "dk", "dv", "dgc", "dgf"), grads):
            assert_close(host64(t[b:b + 1, :, h:h + 1]), g[name], BF16, f"{name} b{b} h{h}")
