"""GPU parity of the forward path (C ABI via the thin binding) against the
fp64 oracle.  Small shapes and every full workload shape are compared
element by element over the whole output (the full shapes run the oracle
one (batch, head) at a time in a thread pool), with the top-K ids checked
on every row; the largest accepted cube count is checked on sampled query
cubes."""
import numpy as np
import pytest
import torch

import oracle
from oracle import vsa_oracle as vo
from tests.gpu_util import (Stats, assert_close, cached_inputs, check_selection, check_selection_row,
                            dev, host64, log, per_head, sum_stats)
from workloads import WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16


def _vsa():
    import trainable_block_sparse_cube_amd as vsa
    return vsa


def unpack_saved(saved, B, nh, N, D):
    """Split the saved buffer by its documented layout (256-byte aligned
    fields): oc [B,nh,Nc,D], lse_c [B,nh,Nc], lse_f [B,nh,N], of [B,nh,N,D]."""
    nc = N // 64
    sizes = [B * nh * nc * D, B * nh * nc, B * nh * N, B * nh * N * D]
    shapes = [(B, nh, nc, D), (B, nh, nc), (B, nh, N), (B, nh, N, D)]
    out, off = [], 0
    raw = saved.view(torch.uint8)
    for n, shp in zip(sizes, shapes):
        out.append(raw[off:off + 4 * n].view(torch.float32).reshape(shp))
        off += (4 * n + 255) // 256 * 256
    return out


def cube_major_to_raster(x_cm, grid):
    """[B, nh, N(cube-major), ...] -> [B, N(raster), nh, ...]."""
    members = vo.cube_members(*grid).ravel()
    out = np.empty_like(x_cm)
    out[:, :, members] = x_cm
    return np.moveaxis(out, 1, 2)


SMALL = [
    # B, heads, D, grid, topk, dtype
    (1, 2, 64, (8, 8, 8), 2, F32),
    (2, 3, 128, (4, 8, 12), 3, BF16),
    (1, 2, 128, (8, 12, 16), 5, BF16),
    (1, 2, 64, (8, 12, 16), 24, BF16),
    (2, 1, 128, (4, 4, 4), 1, BF16),
    (1, 2, 128, (8, 8, 12), 4, F32),
    (1, 3, 64, (12, 8, 16), 7, BF16),
]


def _seeded_shapes(n, seed):
    """n small forward cases drawn once from a fixed seed: grid sides are
    multiples of 4 (1 to 4 cubes per side), 1-2 batches, 1-3 heads, D in
    {64, 128}, K from 1 to all cubes, both dtypes."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        grid = tuple(4 * int(x) for x in rng.integers(1, 5, size=3))
        nc = grid[0] * grid[1] * grid[2] // 64
        out.append((int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.choice([64, 128])), grid,
                    int(rng.integers(1, nc + 1)), F32 if rng.random() < 0.3 else BF16))
    return out


SMALL_SEEDED = _seeded_shapes(10, 2024)


@pytest.mark.parametrize("case", SMALL + SMALL_SEEDED,
                         ids=lambda c: f"B{c[0]}h{c[1]}D{c[2]}g{'x'.join(map(str, c[3]))}k{c[4]}{'f32' if c[5] == F32 else 'bf16'}")
def test_forward_small_full_compare(case):
    B, nh, D, grid, K, dt = case
    log(f"forward small {case}")
    vsa = _vsa()
    inp = make_inputs(B, nh, D, grid, dtype="f32" if dt == F32 else "bf16", seed=100 + K)
    q, k, v, gc, gf = (dev(inp[n], dt) for n in ("q", "k", "v", "gc", "gf"))
    out, sel, saved = vsa.vsa_forward(q, k, v, gc, gf, grid, K, save=True)
    torch.cuda.synchronize()
    sel_np = sel.cpu().numpy()
    ref_own = oracle.forward(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], grid, K)
    check_selection(sel_np, ref_own["S"], K)
    ref = oracle.forward_with_sets(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], grid,
                                   oracle.lists_from_sel(sel_np))
    assert_close(host64(out), ref["o"], dt, "out")
    N = np.prod(grid)
    oc, lse_c, lse_f, of = (host64(t) for t in unpack_saved(saved, B, nh, N, D))
    tol_dt = F32  # saved state is fp32 and compared at the fp32 bar when inputs are fp32
    assert_close(oc, ref["oc"], tol_dt if dt == F32 else BF16, "saved oc")
    np.testing.assert_allclose(lse_c, ref["lse_c"], rtol=0, atol=1e-4)
    assert_close(cube_major_to_raster(of, grid), ref["of"], dt, "saved o_fine")
    np.testing.assert_allclose(np.moveaxis(cube_major_to_raster(lse_f[..., None], grid)[..., 0], 1, 2),
                               ref["lse_f"], rtol=0, atol=2e-3 if dt == BF16 else 1e-4)


@pytest.mark.parametrize("dt", [F32, BF16])
@pytest.mark.parametrize("D", [64, 128])
def test_permute_pool_stage(dt, D):
    vsa = _vsa()
    B, nh, grid = 2, 3, (8, 8, 12)
    log(f"permute_pool {dt} D{D}")
    inp = make_inputs(B, nh, D, grid, dtype="f32" if dt == F32 else "bf16", seed=7)
    q, k, v = (dev(inp[n], dt) for n in "qkv")
    qp, kp, vp, qc, kc, vc = vsa.vsa_cube_permute_pool(q, k, v, grid)
    torch.cuda.synchronize()
    members = vo.cube_members(*grid)  # [Nc, 64]
    for name, x, xp in (("q", inp["q"], qp), ("k", inp["k"], kp), ("v", inp["v"], vp)):
        exp = np.moveaxis(x, 2, 1)[:, :, members]  # [B, nh, Nc, 64, D]
        np.testing.assert_array_equal(xp.float().cpu().numpy(), exp, err_msg=name)
    for name, pooled in (("q", qc), ("k", kc), ("v", vc)):
        exp = np.moveaxis(inp[name].astype(np.float64), 2, 1)[:, :, members].mean(axis=3)
        np.testing.assert_allclose(host64(pooled), exp, rtol=1e-6, atol=1e-6, err_msg=name)


# Coarse-stage bars per product precision.  fp32 products: the fp32 bar.
# bf16 x 3 products (logits to about 2^-16 relative, i.e. about 1e-5 absolute
# on these O(1) logits): Oc still within the fp32 bar and lse_c within 5e-5;
# index parity is unchanged (near-ties are 1e-3 wide).
COARSE_LSE_ATOL = {F32: 1e-5, BF16: 5e-5}


@pytest.mark.parametrize("prec", [F32, BF16], ids=["fp32-products", "bf16x3-products"])
def test_coarse_stage_and_exact_ties(prec):
    """Coarse output and top-K on pooled tensors, including bitwise-equal
    logits made by copying one key cube into another: the lower id wins."""
    vsa = _vsa()
    B, nh, D, grid = 1, 2, 128, (8, 12, 16)  # 24 cubes: a ragged 16-row block
    log("coarse stage")
    inp = make_inputs(B, nh, D, grid, dtype="bf16", seed=31)
    members = vo.cube_members(*grid)
    kk = inp["k"].copy()
    kk[:, members[17]] = kk[:, members[3]]  # key cube 17 := key cube 3
    q, k, v = dev(inp["q"], BF16), dev(kk, BF16), dev(inp["v"], BF16)
    _, _, _, qc, kc, vc = vsa.vsa_cube_permute_pool(q, k, v, grid)
    ref = oracle.forward(inp["q"], kk, inp["v"], inp["gc"], inp["gf"], grid, 1)
    S = ref["S"]
    assert np.array_equal(S[..., 3], S[..., 17])
    straddled = 0
    for K in range(1, 25):
        oc, lse, sel = vsa.vsa_coarse_topk(qc, kc, vc, K, input_dtype=prec)
        torch.cuda.synchronize()
        sel_np = sel.cpu().numpy()
        check_selection(sel_np, S, K)
        for b, h, r in np.ndindex(B, nh, 24):
            order = np.lexsort((np.arange(24), -S[b, h, r]))
            if order[K - 1] == 3 and order[K] == 17:  # the tie sits on the boundary
                straddled += 1
                assert 3 in sel_np[b, h, r] and 17 not in sel_np[b, h, r]
        if K == 5:
            assert_close(host64(oc), ref["oc"], F32, "oc")  # the fp32 bar in both precisions
            np.testing.assert_allclose(host64(lse), ref["lse_c"], atol=COARSE_LSE_ATOL[prec])
    assert straddled > 0


@pytest.mark.parametrize("D,grid", [(128, (8, 12, 20)), (64, (8, 36, 44)), (128, (4, 40, 48)),
                                   (64, (4, 32, 1200))],
                         ids=["D128-30cubes", "D64-198cubes", "D128-120cubes", "D64-2400cubes"])
def test_forward_coarse_packed_equals_stage_call(D, grid):
    """The bf16 forward hands the coarse kernel its pooled K and V in packed
    operand order (padding keys zeroed); the stage call reads plain means.
    Same products in the same order, so the saved coarse output and LSE and
    the selection agree bitwise, also with cube counts that leave ragged
    16- and 32-key blocks."""
    vsa = _vsa()
    B, nh, K = 1, 2, 6
    T, H, W = grid
    N = T * H * W
    log(f"packed coarse vs stage call D={D} grid={grid}")
    inp = make_inputs(B, nh, D, grid, dtype="bf16", seed=77)
    q, k, v, gc, gf = (dev(inp[n], BF16) for n in ("q", "k", "v", "gc", "gf"))
    out, sel, saved = vsa.vsa_forward(q, k, v, gc, gf, grid, K, save=True)
    _, _, _, qc, kc, vc = vsa.vsa_cube_permute_pool(q, k, v, grid, with_q_tiles=False)
    oc, lse, sel2 = vsa.vsa_coarse_topk(qc, kc, vc, K, input_dtype=BF16)
    torch.cuda.synchronize()
    oc_s, lse_s, _, _ = unpack_saved(saved, B, nh, N, D)
    assert torch.equal(sel, sel2)
    assert torch.equal(oc_s, oc)
    assert torch.equal(lse_s, lse)


@pytest.mark.parametrize("prec", [F32, BF16], ids=["fp32-products", "bf16x3-products"])
@pytest.mark.parametrize("grid,n_cubes", [((4, 32, 1792), 3584), ((4, 32, 1200), 2400),
                                           ((4, 36, 1012), 2277), ((4, 32, 1136), 2272),
                                           ((4, 32, 548), 1096), ((4, 32, 600), 1200)],
                         ids=["3584cubes", "2400cubes", "2277cubes", "2272cubes", "1096cubes",
                              "1200cubes"])
def test_coarse_stage_at_large_cube_counts(prec, grid, n_cubes):
    """3584 cubes (grid 4x32x1792), the most the coarse kernel holds (8 rows
    of logits in LDS, 56 key chunks of 64 per row in registers); 2400 cubes
    (8 rows, 40 chunks); 2277 cubes (8 rows, the last block holding 5);
    2272 cubes, the most with 16 rows; 1096 cubes (20
    chunks per row, two workgroups per CU with 128 ranking candidates per
    wave) and 1200 cubes (20 chunks, 256 candidates, one workgroup per CU):
    top-K 32 (pruned candidate ranking),
    100 (bitwise search) and all cubes, plus the mass rule (long lists, more
    candidates than the scratch holds)."""
    from tests.gpu_util import check_mass_row
    vsa = _vsa()
    log(f"coarse stage at {n_cubes} cubes, {prec}")
    inp = make_inputs(1, 1, 128, grid, dtype="bf16", seed=41)
    q, k, v = (dev(inp[n], BF16) for n in "qkv")
    _, _, _, qc, kc, vc = vsa.vsa_cube_permute_pool(q, k, v, grid, with_q_tiles=False)
    nc = qc.shape[2]
    assert nc == n_cubes
    pooled = [vo.pool(inp[n][0, :, 0].astype(np.float64), *grid) for n in "qkv"]
    oc_ref, S, lse_ref = vo.coarse_attention(*pooled, 1.0 / np.sqrt(128))
    for K in (32, 100, nc):
        oc, lse, sel = vsa.vsa_coarse_topk(qc, kc, vc, K, input_dtype=prec)
        torch.cuda.synchronize()
        check_selection(sel.cpu().numpy(), S[None, None], K)
    assert_close(host64(oc)[0, 0], oc_ref, F32, "oc")
    np.testing.assert_allclose(host64(lse)[0, 0], lse_ref, atol=COARSE_LSE_ATOL[prec])
    mass, k_min, k_max = 0.3, 4, 96
    _, _, counts, ids = vsa.vsa_coarse_select_mass(qc, kc, vc, mass, k_min, k_max, input_dtype=prec)
    torch.cuda.synchronize()
    counts, ids = counts.cpu().numpy()[0, 0], ids.cpu().numpy()[0, 0]
    banded = 0
    for r in range(0, nc, 7):  # every 7th row against the fp64 logits
        n = int(counts[r])
        assert k_min <= n <= k_max
        banded += not check_mass_row(ids[r][:n], S[r], mass, k_min, k_max)
    assert banded <= 2


def test_coarse_topk_zero_skips_selection():
    vsa = _vsa()
    inp = make_inputs(1, 1, 64, (4, 8, 8), dtype="f32", seed=2)
    q, k, v = (dev(inp[n], F32) for n in "qkv")
    _, _, _, qc, kc, vc = vsa.vsa_cube_permute_pool(q, k, v, (4, 8, 8))
    oc, lse, sel = vsa.vsa_coarse_topk(qc, kc, vc, 0)
    torch.cuda.synchronize()
    assert sel is None
    ref = oracle.forward(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], (4, 8, 8), 1)
    assert_close(host64(oc), ref["oc"], F32, "oc")


def test_dense_topk_equals_library_attention():
    """K = Nc: the fine stage is dense attention (torch SDPA in fp32 on the
    same bf16 inputs), checked with the gates set to (0, 1)."""
    vsa = _vsa()
    B, nh, D, grid = 1, 2, 128, (8, 8, 8)  # 8 cubes
    inp = make_inputs(B, nh, D, grid, dtype="bf16", seed=3)
    q, k, v = (dev(inp[n], BF16) for n in "qkv")
    zero = torch.zeros(B, 512, nh, dtype=BF16, device="cuda")
    one = torch.ones_like(zero)
    out, sel, _ = vsa.vsa_forward(q, k, v, zero, one, grid, 8)
    torch.cuda.synchronize()
    assert np.all(sel.cpu().numpy() == np.arange(8))
    qf, kf, vf = (t.float().permute(0, 2, 1, 3).contiguous() for t in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qf, kf, vf).permute(0, 2, 1, 3)
    assert_close(host64(out), host64(ref), BF16, "dense")


@pytest.mark.parametrize("dt", [F32, BF16])
def test_varlen_small_including_empty_and_full_lists(dt):
    vsa = _vsa()
    B, nh, D, grid = 2, 2, 64, (8, 8, 12)  # 12 cubes
    log(f"varlen small {dt}")
    inp = make_inputs(B, nh, D, grid, dtype="f32" if dt == F32 else "bf16", seed=8, varlen=(0, 12))
    offs, ids = inp["kv_offsets"].copy(), inp["kv_ids"].copy()
    counts = np.diff(offs)
    assert (counts == 0).any() and (counts == 12).any()
    q, k, v, gc, gf = (dev(inp[n], dt) for n in ("q", "k", "v", "gc", "gf"))
    out, saved = vsa.block_sparse_attn_varlen(q, k, v, gc, gf, grid,
                                              torch.from_numpy(offs).cuda(), torch.from_numpy(ids).cuda(),
                                              save=True)
    torch.cuda.synchronize()
    lists = oracle.lists_from_csr(offs, ids, B, nh, 12)
    ref = oracle.forward_with_sets(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], grid, lists)
    assert_close(host64(out), ref["o"], dt, "varlen out")
    lse_f = host64(unpack_saved(saved, B, nh, 768, D)[2])
    members = vo.cube_members(*grid)
    for r, cnt in enumerate(counts):
        if cnt == 0:
            b, h, c = r // (nh * 12), (r // 12) % nh, r % 12
            assert np.all(np.isneginf(lse_f[b, h, c * 64:(c + 1) * 64]))
            np.testing.assert_allclose(host64(out)[b, members[c], h], ref["o"][b, members[c], h], atol=2e-2)


def test_varlen_with_topk_lists_reproduces_vsa_forward():
    vsa = _vsa()
    B, nh, D, grid, K = 1, 2, 128, (8, 8, 12), 3
    inp = make_inputs(B, nh, D, grid, dtype="bf16", seed=9)
    q, k, v, gc, gf = (dev(inp[n], BF16) for n in ("q", "k", "v", "gc", "gf"))
    out, sel, _ = vsa.vsa_forward(q, k, v, gc, gf, grid, K)
    offs = torch.arange(0, B * nh * 12 * K + 1, K, dtype=torch.int32, device="cuda")
    out2, _ = vsa.block_sparse_attn_varlen(q, k, v, gc, gf, grid, offs, sel.reshape(-1).contiguous())
    shuffled = sel.flip(-1).reshape(-1).contiguous()  # order inside a list is free
    out3, _ = vsa.block_sparse_attn_varlen(q, k, v, gc, gf, grid, offs, shuffled)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert_close(host64(out3), host64(out), BF16, "shuffled lists")


def _order_key(p1, p3, nc):
    """The processing order's sort key: the list entries at a quarter and
    at three quarters, each scaled to 9 bits (id * 512 // Nc), as a Morton
    code with the first point's bits above the second's."""
    x = (np.asarray(p1, dtype=np.int64) << 9) // nc
    y = (np.asarray(p3, dtype=np.int64) << 9) // nc
    key = np.zeros_like(x)
    for j in range(9):
        key |= ((x >> j) & 1) << (2 * j + 1)
        key |= ((y >> j) & 1) << (2 * j)
    return key


def _want_order(keys):
    """keys [n_bh, nc]: ascending key, cube index on ties, as global ids."""
    n_bh, nc = keys.shape
    return np.concatenate([bh * nc + np.lexsort((np.arange(nc), keys[bh])) for bh in range(n_bh)])


def test_order_key_model():
    """The test's model of the sort key on hand-worked values (Nc = 512, so
    ids are their own 9-bit coordinates): the first point's bits land on
    the odd positions."""
    assert _order_key([1], [0], 512)[0] == 0b10
    assert _order_key([0], [1], 512)[0] == 0b01
    assert _order_key([3], [5], 512)[0] == 0b11011  # x = 0b011 on bits 1, 3; y = 0b101 on bits 0, 4
    assert _order_key([511], [511], 512)[0] == (1 << 18) - 1
    assert _order_key([959], [480], 960)[0] == _order_key([511], [256], 512)[0]  # 959 * 512 // 960 = 511


def test_fine_order_sorts_by_quartile_entries_and_changes_nothing():
    """The fine stage's processing order: each (b, h)'s query cubes sorted by
    the Morton code of their lists' entries at indices n/4 and 3n/4, cube
    index on ties (exact), for fixed and CSR lists with empty ones; running
    in that order leaves the output bitwise unchanged."""
    vsa = _vsa()
    B, nh, D, grid, K = 2, 3, 128, (8, 12, 16), 5  # 24 cubes
    nc = 24
    inp = make_inputs(B, nh, D, grid, dtype="bf16", seed=62, varlen=(0, 24))
    q, k, v, gc, gf = (dev(inp[n], BF16) for n in ("q", "k", "v", "gc", "gf"))
    _, kp, vp, qc, kc, vc = vsa.vsa_cube_permute_pool(q, k, v, grid, with_q_tiles=False)
    oc, _, sel = vsa.vsa_coarse_topk(qc, kc, vc, K, input_dtype=BF16)
    order = vsa.vsa_fine_order(sel, B, nh, nc, topk=K)
    torch.cuda.synchronize()
    s3 = sel.cpu().numpy().reshape(B * nh, nc, K)
    np.testing.assert_array_equal(order.cpu().numpy(),
                                  _want_order(_order_key(s3[:, :, K // 4], s3[:, :, (3 * K) // 4], nc)))
    out0, _, _ = vsa.vsa_fine_forward(q, kp, vp, oc, gc, gf, grid, sel, topk=K)
    out1, _, _ = vsa.vsa_fine_forward(q, kp, vp, oc, gc, gf, grid, sel, topk=K, order=order)
    torch.cuda.synchronize()
    assert torch.equal(out0, out1)
    offs, ids = inp["kv_offsets"], inp["kv_ids"]
    assert (np.diff(offs) == 0).any() and (np.diff(offs) == 1).any()
    order = vsa.vsa_fine_order(torch.from_numpy(ids).cuda(), B, nh, nc,
                               kv_offsets=torch.from_numpy(offs).cuda())
    torch.cuda.synchronize()
    n = np.diff(offs)
    p1 = np.where(n > 0, ids[np.minimum(offs[:-1] + n // 4, len(ids) - 1)], 0)
    p3 = np.where(n > 0, ids[np.minimum(offs[:-1] + (3 * n) // 4, len(ids) - 1)], 0)
    keys = np.where(n > 0, _order_key(p1, p3, nc), 0).reshape(B * nh, nc)
    np.testing.assert_array_equal(order.cpu().numpy(), _want_order(keys))
    # larger (b, h) blocks, drawn directly: random sorted lists up to the
    # sort's 4096-cube limit, and identical lists (one bucket of every cube)
    rng = np.random.default_rng(64)
    for n_bh, nc, K, same in ((3, 512, 16, False), (2, 4096, 32, False), (2, 960, 32, True), (2, 960, 1, False)):
        if same:
            lists = np.broadcast_to(np.arange(K, dtype=np.int32), (n_bh * nc, K))
        else:
            lists = np.sort(np.stack([rng.choice(nc, K, replace=False) for _ in range(n_bh * nc)]), axis=1)
        lists = np.ascontiguousarray(lists, dtype=np.int32)
        order = vsa.vsa_fine_order(torch.from_numpy(lists).cuda(), 1, n_bh, nc, topk=K)
        torch.cuda.synchronize()
        l3 = lists.reshape(n_bh, nc, K)
        np.testing.assert_array_equal(order.cpu().numpy(),
                                      _want_order(_order_key(l3[:, :, K // 4], l3[:, :, (3 * K) // 4], nc)))


def test_fine_order_entries_out_of_range_run_nothing():
    """An order entry outside [0, B*heads*Nc) runs no cube (the kernel's own
    range check): those cubes' rows keep what the output held, every other
    row equals the natural-order result."""
    vsa = _vsa()
    B, nh, D, grid, K = 1, 2, 128, (8, 12, 16), 5  # 24 cubes per head
    nc = 24
    inp = make_inputs(B, nh, D, grid, dtype="bf16", seed=63)
    q, k, v, gc, gf = (dev(inp[n], BF16) for n in ("q", "k", "v", "gc", "gf"))
    _, kp, vp, qc, kc, vc = vsa.vsa_cube_permute_pool(q, k, v, grid, with_q_tiles=False)
    oc, _, sel = vsa.vsa_coarse_topk(qc, kc, vc, K, input_dtype=BF16)
    ref, _, _ = vsa.vsa_fine_forward(q, kp, vp, oc, gc, gf, grid, sel, topk=K)
    order = torch.arange(B * nh * nc, dtype=torch.int32, device="cuda")
    dropped = [3, nc + 7]
    order[dropped[0]] = -1
    order[dropped[1]] = B * nh * nc
    out = torch.full_like(q, float("nan"))
    vsa.vsa_fine_forward(q, kp, vp, oc, gc, gf, grid, sel, topk=K, out=out, order=order)
    torch.cuda.synchronize()
    # token rows of each dropped cube (raster order), for its head
    T, H, W = grid
    cube_rows = {}
    for g in dropped:
        h, c = divmod(g, nc)
        W4, H4 = W // 4, H // 4
        ct, cy, cx = c // (H4 * W4), (c // W4) % H4, c % W4
        toks = [((4 * ct + s // 16) * H + 4 * cy + (s // 4) % 4) * W + 4 * cx + s % 4 for s in range(64)]
        cube_rows[g] = (h, toks)
    o, r = out.float().cpu(), ref.float().cpu()
    mask = torch.zeros(o.shape[:3], dtype=torch.bool)
    for g, (h, toks) in cube_rows.items():
        mask[0, toks, h] = True
    assert torch.isnan(o[mask]).all()
    assert torch.equal(o[~mask], r[~mask])


def test_forward_is_deterministic():
    vsa = _vsa()
    grid = (8, 16, 16)
    inp = make_inputs(1, 4, 128, grid, dtype="bf16", seed=10)
    args = [dev(inp[n], BF16) for n in ("q", "k", "v", "gc", "gf")]
    o1, s1, _ = vsa.vsa_forward(*args, grid, 6, save=True)
    o2, s2, _ = vsa.vsa_forward(*args, grid, 6, save=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_mass_and_varlen_paths_are_deterministic():
    """The mass-rule forward (coarse rule, CSR packing, sorted fine stage)
    and the varlen forward and backward give bitwise-equal results when
    called twice on the same inputs."""
    vsa = _vsa()
    grid = (8, 16, 16)
    inp = make_inputs(2, 3, 128, grid, dtype="bf16", seed=12, with_dout=True)
    args = [dev(inp[n], BF16) for n in ("q", "k", "v", "gc", "gf")]
    do = dev(inp["dout"], BF16)
    runs = [vsa.vsa_forward_mass(*args, grid, 0.3, 2, 20, save=True) for _ in range(2)]
    torch.cuda.synchronize()
    (o1, f1, i1, _), (o2, f2, i2, _) = runs
    assert torch.equal(f1, f2) and torch.equal(i1, i2) and torch.equal(o1, o2)
    out1, sv1 = vsa.block_sparse_attn_varlen(*args, grid, f1, i1, save=True)
    out2, sv2 = vsa.block_sparse_attn_varlen(*args, grid, f1, i1, save=True)
    g1 = vsa.block_sparse_attn_varlen_backward(*args, do, f1, i1, sv1, grid)
    g2 = vsa.block_sparse_attn_varlen_backward(*args, do, f1, i1, sv2, grid)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(out1, o1)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


# --------------------------------------------------------------- full sizes
def _sampled_check(w, inp, out, sel_np, K, n_samples, rng, lists=None):
    B, nh, D = w.B, w.heads, w.head_dim
    nc = w.n_cubes
    exempt = 0
    outs, refs = [], []
    for _ in range(n_samples):
        b, h, c = int(rng.integers(B)), int(rng.integers(nh)), int(rng.integers(nc))
        ids = lists(b, h, c) if lists else sel_np[b, h, c]
        rows, o_ref, _, logits = oracle.query_cube_output(
            inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], w.grid, b, h, c, ids)
        if lists is None and not check_selection_row(sel_np[b, h, c], logits, K):
            exempt += 1
        o_gpu = out[b, torch.from_numpy(rows).cuda(), h].float().cpu().numpy()
        outs.append(o_gpu); refs.append(o_ref)
    assert_close(np.stack(outs), np.stack(refs), BF16, f"{w.name} sampled rows")
    return exempt


def test_forward_at_the_largest_cube_count():
    """3584 cubes per (batch, head) (grid 4x32x1792, head_dim 64, 2 heads),
    the most the library accepts: the processing-order sort at its largest
    size (4096 keys), the coarse stage with 8-row workgroups and 56-chunk
    rows on packed means, and the fine stage.  Every row's ids valid, and
    sampled query cubes against the oracle one by one."""
    import types
    vsa = _vsa()
    grid, B, nh, D, K = (4, 32, 1792), 1, 2, 64, 32
    w = types.SimpleNamespace(name="3584cubes", B=B, heads=nh, head_dim=D, n_cubes=3584, grid=grid)
    log("forward at 3584 cubes: drawing inputs")
    inp = make_inputs(B, nh, D, grid, dtype="bf16", seed=91)
    q, k, v, gc, gf = (dev(inp[n], BF16) for n in ("q", "k", "v", "gc", "gf"))
    out, sel, _ = vsa.vsa_forward(q, k, v, gc, gf, grid, K)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())
    sel_np = sel.cpu().numpy()
    assert sel_np.shape == (B, nh, 3584, K)
    assert np.all(np.diff(sel_np, axis=-1) > 0) and sel_np.min() >= 0 and sel_np.max() < 3584
    exempt = _sampled_check(w, inp, out, sel_np, K, 8, np.random.default_rng(5))
    log(f"  3584 cubes: sampled rows ok, near-tie exemptions {exempt}/8")


def _whole_forward_check(w, inp, o_np, lists_of, sel_np=None, K=None):
    """Per (b, h), in a thread pool: the oracle forward under the GPU's
    lists (or the caller's), compared over the whole head; with sel_np, the
    ids of every row are checked against the oracle's fp64 logits.
    Returns (Stats over the whole output, near-tie exemptions)."""
    def work(b, h):
        sl = lambda n: inp[n][b:b + 1, :, h:h + 1]
        r = oracle.forward_with_sets(sl("q"), sl("k"), sl("v"), sl("gc"), sl("gf"), w.grid,
                                     [[lists_of(b, h)]])
        exempt = check_selection(sel_np[b, h][None], r["S"][0], K) if sel_np is not None else 0
        return Stats.of(o_np[b, :, h], r["o"][0, :, 0]), exempt
    res = per_head(work, [(b, h) for b in range(w.B) for h in range(w.heads)])
    return sum_stats(r[0] for r in res), sum(r[1] for r in res)


# large70k last, so that the varlen test below reuses its drawn inputs
@pytest.mark.parametrize("name,K", [("pretrain16k", 32), ("train16k", 32), ("long61k_smooth", 32),
                                    ("long61k", 16), ("long61k", 32), ("large70k", 32)])
def test_forward_full_size_whole_tensor(name, K):
    """Every workload shape at full size: the output starts as NaN (so an
    unwritten row cannot pass), then the whole tensor is compared with the
    oracle under the GPU's own selection, and every row's ids with the
    oracle's fp64 coarse logits (near-tie rule)."""
    vsa = _vsa()
    w = WORKLOADS[name]
    log(f"full-size forward {name} K={K}: drawing inputs")
    inp = cached_inputs(name, w.varlen is not None)
    q, k, v, gc, gf = (dev(inp[n], BF16) for n in ("q", "k", "v", "gc", "gf"))
    out = torch.full_like(q, float("nan"))
    log(f"full-size forward {name} K={K}: running")
    _, sel, _ = vsa.vsa_forward(q, k, v, gc, gf, w.grid, K, out=out)
    torch.cuda.synchronize()
    sel_np = sel.cpu().numpy()
    o_np = out.float().cpu().numpy()
    del q, k, v, gc, gf, out
    assert np.all(np.diff(sel_np, axis=-1) > 0) and sel_np.min() >= 0 and sel_np.max() < w.n_cubes
    log(f"full-size forward {name} K={K}: oracle on {w.B * w.heads} heads")
    st, exempt = _whole_forward_check(w, inp, o_np, lambda b, h: list(sel_np[b, h]), sel_np, K)
    msg = st.check(BF16, f"{name} K={K} whole output")
    log(f"  {msg}; near-tie rows {exempt}/{sel_np.shape[0] * sel_np.shape[1] * sel_np.shape[2]}")


def test_varlen_full_size_whole_tensor():
    """large70k with per-query-cube lists of 8..64 random cubes: whole
    output against the oracle under the same lists."""
    vsa = _vsa()
    w = WORKLOADS["large70k"]
    log("full-size varlen large70k: drawing inputs")
    inp = cached_inputs("large70k", True)
    offs, ids = inp["kv_offsets"], inp["kv_ids"]
    q, k, v, gc, gf = (dev(inp[n], BF16) for n in ("q", "k", "v", "gc", "gf"))
    out = torch.full_like(q, float("nan"))
    vsa.block_sparse_attn_varlen(q, k, v, gc, gf, w.grid, torch.from_numpy(offs).cuda(),
                                 torch.from_numpy(ids).cuda(), out=out)
    torch.cuda.synchronize()
    o_np = out.float().cpu().numpy()
    del q, k, v, gc, gf, out
    nc = w.n_cubes

    def lists_of(b, h):
        r0 = (b * w.heads + h) * nc
        return [ids[offs[r0 + c]:offs[r0 + c + 1]] for c in range(nc)]
    log("full-size varlen large70k: oracle")
    st, _ = _whole_forward_check(w, inp, o_np, lists_of)
    log("  " + st.check(BF16, "large70k varlen whole output"))
