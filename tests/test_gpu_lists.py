"""Validation of caller-made key lists on the GPU (include/vsa.h,
vsa_validate_lists, and VSA_VALIDATE=1): well-formed lists pass, and each
kind of malformed list is counted.  The check kernel only reads and compares
list values, so malformed lists are safe to hand it; they are never handed
to the attention kernels here."""
import os

import numpy as np
import pytest
import torch

from tests.gpu_util import dev, log
from workloads import make_inputs

pytestmark = pytest.mark.gpu


def _vsa():
    import trainable_block_sparse_cube_amd as vsa
    return vsa


def _csr(lists):
    offs = np.zeros(len(lists) + 1, dtype=np.int32)
    offs[1:] = np.cumsum([len(x) for x in lists])
    ids = np.concatenate([np.asarray(x, dtype=np.int32) for x in lists]) if offs[-1] else np.zeros(0, np.int32)
    return torch.from_numpy(offs).cuda(), torch.from_numpy(ids.astype(np.int32)).cuda()


def _good_lists(n_rows, nc, rng, lo=0):
    return [np.sort(rng.choice(nc, int(rng.integers(lo, min(9, nc + 1))), replace=False))
            for _ in range(n_rows)]


def test_well_formed_lists_pass():
    vsa = _vsa()
    rng = np.random.default_rng(1)
    for nc in (8, 100, 3584):
        lists = _good_lists(200, nc, rng)
        offs, ids = _csr(lists)
        assert vsa.validate_lists(ids, 200, nc, kv_offsets=offs) == (0, 0)
        # fixed length (top-K style): all rows distinct ids
        sel = np.stack([rng.choice(nc, 5, replace=False) for _ in range(50)]).astype(np.int32)
        assert vsa.validate_lists(torch.from_numpy(sel).cuda(), 50, nc, topk=5) == (0, 0)
    # no rows with entries at all
    offs, ids = _csr([[] for _ in range(7)])
    assert vsa.validate_lists(torch.zeros(0, dtype=torch.int32, device="cuda"), 7, 8, kv_offsets=offs) == (0, 0)
    # an id array longer than the offsets say is an offset fault (the end is checked)
    assert vsa.validate_lists(torch.zeros(1, dtype=torch.int32, device="cuda"), 7, 8, kv_offsets=offs) == (1, 0)


def test_each_malformation_is_counted():
    vsa = _vsa()
    rng = np.random.default_rng(2)
    nc, n_rows = 64, 40
    lists = _good_lists(n_rows, nc, rng)
    lists[3] = [1, 5, 9]
    lists[4] = [2, 2, 7]        # repeated id
    lists[10] = [0, nc]          # id out of range (= Nc)
    lists[11] = [-1]             # negative id
    offs, ids = _csr(lists)
    assert vsa.validate_lists(ids, n_rows, nc, kv_offsets=offs) == (0, 3)
    good = _good_lists(n_rows, nc, rng, lo=1)   # every list non-empty: offsets strictly increase
    offs, ids = _csr(good)
    o = offs.clone(); o[0] = 1            # does not start at 0 (and row 0 shrinks: still readable)
    assert vsa.validate_lists(ids, n_rows, nc, kv_offsets=o)[0] >= 1
    o = offs.clone(); o[-1] = o[-1] - 1                             # end != number of ids
    assert vsa.validate_lists(ids, n_rows, nc, kv_offsets=o)[0] >= 1
    o = offs.clone(); o[6] = int(offs[5]) - 1                       # a decrease
    assert vsa.validate_lists(ids, n_rows, nc, kv_offsets=o)[0] >= 1
    # fixed length with a repeat and an out-of-range id
    sel = np.stack([rng.choice(nc, 4, replace=False) for _ in range(10)]).astype(np.int32)
    sel[2, 1] = sel[2, 0]
    sel[7, 3] = 1000
    assert vsa.validate_lists(torch.from_numpy(sel).cuda(), 10, nc, topk=4) == (0, 2)


def test_binding_and_env_check_reject_bad_lists_before_attention():
    """The binding's default check raises before anything else is queued;
    with validate=False and VSA_VALIDATE=1 the library's own check refuses
    the call with VSA_ERR_INVALID_ARG.  Well-formed lists still run."""
    vsa = _vsa()
    from trainable_block_sparse_cube_amd import _lib
    grid, nh = (4, 8, 8), 2           # 8 cubes
    inp = make_inputs(1, nh, 64, grid, dtype="bf16", seed=3)
    q, k, v, gc, gf = (dev(inp[n], torch.bfloat16) for n in ("q", "k", "v", "gc", "gf"))
    rng = np.random.default_rng(4)
    lists = _good_lists(nh * 4, 4, rng)
    bad = list(lists)
    bad[1] = [0, 0]
    offs, ids = _csr(bad)
    with pytest.raises(ValueError, match="malformed key lists"):
        vsa.block_sparse_attn_varlen(q, k, v, gc, gf, grid, offs, ids)
    old = os.environ.get("VSA_VALIDATE")
    os.environ["VSA_VALIDATE"] = "1"
    try:
        with pytest.raises(_lib.VSAError) as e:
            vsa.block_sparse_attn_varlen(q, k, v, gc, gf, grid, offs, ids, validate=False)
        assert e.value.status == _lib.VSA_ERR_INVALID_ARG
        goffs, gids = _csr(lists)
        out, _ = vsa.block_sparse_attn_varlen(q, k, v, gc, gf, grid, goffs, gids, validate=False)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out.float()).all())
    finally:
        if old is None:
            del os.environ["VSA_VALIDATE"]
        else:
            os.environ["VSA_VALIDATE"] = old
    log("  malformed lists refused before the attention kernels")
