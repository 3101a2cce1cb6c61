"""Pins for the fp64 oracle, each against something other than the oracle:
library dense attention (torch fp64 SDPA), index maps built by reshape,
brute-force scalar loops, closed forms, invariants and central finite
differences.  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import vsa_oracle as vo
from workloads import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sdpa64(q, k, v):
    """Dense softmax attention from torch's library routine, fp64 CPU."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))[0, 0].numpy()


def small(B=1, nh=2, D=16, grid=(4, 8, 12), seed=7, dtype="f32"):
    return make_inputs(B, nh, D, grid, dtype=dtype, seed=seed, with_dout=True)


# ---------------------------------------------------------------- step 1: cubes
@pytest.mark.parametrize("grid", [(4, 4, 4), (4, 8, 12), (8, 4, 16), (12, 8, 8)])
def test_cube_members_match_reshape_order(grid):
    T, H, W = grid
    ref = (np.arange(T * H * W).reshape(T // 4, 4, H // 4, 4, W // 4, 4)
           .transpose(0, 2, 4, 1, 3, 5).reshape(-1, 64))
    np.testing.assert_array_equal(vo.cube_members(T, H, W), ref)
    cube, slot = vo.token_cube_map(T, H, W)
    # bijection tokens <-> (cube, slot)
    assert np.unique(cube * 64 + slot).size == T * H * W


def test_cube_map_hand_values():
    # 4x4x8 grid: two cubes along x.  token (0,0,4) -> cube 1 slot 0;
    # token (3,3,7) -> cube 1 slot 63; token (1,2,3) -> cube 0 slot 16+8+3.
    cube, slot = vo.token_cube_map(4, 4, 8)
    tok = lambda t, y, x: (t * 4 + y) * 8 + x
    assert (cube[tok(0, 0, 4)], slot[tok(0, 0, 4)]) == (1, 0)
    assert (cube[tok(3, 3, 7)], slot[tok(3, 3, 7)]) == (1, 63)
    assert (cube[tok(1, 2, 3)], slot[tok(1, 2, 3)]) == (0, 27)


def test_grid_not_divisible_rejected():
    with pytest.raises(ValueError):
        vo.token_cube_map(4, 6, 8)


# ---------------------------------------------------------------- step 2: pool
def test_pool_cube_constant_exact_and_sum_invariant():
    T, H, W = 8, 4, 8
    rng = np.random.default_rng(0)
    vals = rng.integers(-64, 64, size=(4, 3)) / 8.0  # few mantissa bits: sums are exact
    cube, _ = vo.token_cube_map(T, H, W)
    x = vals[cube]
    np.testing.assert_array_equal(vo.pool(x, T, H, W), vals)
    y = rng.standard_normal((T * H * W, 5))
    np.testing.assert_allclose((64 * vo.pool(y, T, H, W)).sum(0), y.sum(0), rtol=1e-12, atol=1e-12)


def _max_pool_by_reshape(x, T, H, W):
    """Per-cube channel max built from a reshape of the grid, independent of
    the oracle's member table."""
    D = x.shape[-1]
    g = x.reshape(T // 4, 4, H // 4, 4, W // 4, 4, D)
    return g.max(axis=(1, 3, 5)).reshape(-1, D)


def test_max_pool_matches_reshape_and_bounds_mean():
    T, H, W = 8, 12, 8
    rng = np.random.default_rng(1)
    y = rng.standard_normal((T * H * W, 6))
    mx = vo.pool(y, T, H, W, op="max")
    np.testing.assert_array_equal(mx, _max_pool_by_reshape(y, T, H, W))
    assert np.all(mx >= vo.pool(y, T, H, W))
    vals = rng.standard_normal((vo.cube_members(T, H, W).shape[0], 6))
    cube, _ = vo.token_cube_map(T, H, W)
    np.testing.assert_array_equal(vo.pool(vals[cube], T, H, W, op="max"), vals)
    with pytest.raises(ValueError):
        vo.pool(y, T, H, W, op="median")


def test_cube_attention_mass_against_library_softmax():
    from scipy.special import softmax
    T, H, W = 8, 8, 12  # 12 cubes
    inp = small(nh=2, D=16, seed=4, grid=(T, H, W))
    cube, _ = vo.token_cube_map(T, H, W)
    members = vo.cube_members(T, H, W)
    for b, h, c in ((0, 0, 0), (0, 1, 7), (0, 1, 11)):
        m = vo.cube_attention_mass(inp["q"], inp["k"], (T, H, W), b, h, c)
        assert abs(m.sum() - 1.0) < 1e-12 and np.all(m > 0)
        Q = inp["q"][b, members[c], h].astype(np.float64)
        K = inp["k"][b, :, h].astype(np.float64)
        w = softmax(np.einsum("id,jd->ij", Q, K) / 4.0, axis=1)  # 1/sqrt(16)
        want = np.bincount(cube, weights=w.mean(axis=0), minlength=12)
        np.testing.assert_allclose(m, want, rtol=1e-12, atol=1e-15)
    k = inp["k"].copy()
    k[:] = k[:, :1]  # every key identical: every cube gets 1/Nc
    np.testing.assert_allclose(vo.cube_attention_mass(inp["q"], k, (T, H, W), 0, 0, 3), np.full(12, 1 / 12),
                               rtol=1e-12)


# ---------------------------------------------------------------- step 3: coarse
def test_coarse_equals_library_attention_on_pooled():
    inp = small()
    T, H, W = 4, 8, 12
    q, k, v = (inp[n][0, :, 1].astype(np.float64) for n in "qkv")
    qc, kc, vc = (vo.pool(x, T, H, W) for x in (q, k, v))
    oc, S, lse = vo.coarse_attention(qc, kc, vc, 1 / math.sqrt(16))
    np.testing.assert_allclose(oc, sdpa64(qc, kc, vc), rtol=1e-12, atol=1e-12)
    from scipy.special import logsumexp
    np.testing.assert_allclose(lse, logsumexp(S, axis=1), rtol=1e-13, atol=1e-13)
    # the forward's coarse output is the same thing
    r = oracle.forward(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], (T, H, W), 2)
    np.testing.assert_allclose(r["oc"][0, 1], sdpa64(qc, kc, vc), rtol=1e-12, atol=1e-12)


def test_coarse_uniform_keys_average_values():
    rng = np.random.default_rng(1)
    qc = rng.standard_normal((6, 8)); vc = rng.standard_normal((6, 8))
    kc = np.tile(rng.standard_normal((1, 8)), (6, 1))
    oc, _, _ = vo.coarse_attention(qc, kc, vc, 0.3)
    np.testing.assert_allclose(oc, np.tile(vc.mean(0), (6, 1)), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- top-K
def _rank_select(S, K):
    """Selection by counting: j is chosen iff fewer than K cubes beat it,
    where i beats j when S[i] > S[j], or S[i] == S[j] and i < j."""
    nc = S.shape[1]
    out = []
    for row in S:
        chosen = [j for j in range(nc)
                  if sum(1 for i in range(nc) if row[i] > row[j] or (row[i] == row[j] and i < j)) < K]
        out.append(chosen)
    return np.array(out)


@pytest.mark.parametrize("K", [1, 3, 7, 12])
def test_topk_matches_counting_definition(K):
    rng = np.random.default_rng(K)
    S = rng.standard_normal((9, 12))
    S[:, 5] = S[:, 2]  # exact ties
    S[3, :] = 0.25  # a fully tied row
    sel = vo.select_topk(S, K)
    np.testing.assert_array_equal(sel, _rank_select(S, K))
    for r in range(S.shape[0]):
        assert len(set(sel[r])) == K and np.all(np.diff(sel[r]) > 0)
        rest = np.setdiff1d(np.arange(12), sel[r])
        if rest.size:
            assert S[r, sel[r]].min() >= S[r, rest].max()
    np.testing.assert_array_equal(sel[3], np.arange(K))


def test_topk_rejects_bad_k():
    with pytest.raises(ValueError):
        vo.select_topk(np.zeros((2, 4)), 0)
    with pytest.raises(ValueError):
        vo.select_topk(np.zeros((2, 4)), 5)


# ------------------------------------------- step 3': stand-in mass rule
def _softmax_lib(row):
    from scipy.special import softmax
    return softmax(row)


def _check_mass_list(row, ids, mass, k_min, k_max):
    """Invariants of one list of the mass rule, independent of its code:
    ascending distinct ids; every chosen logit >= every unchosen one, equal
    logits going to the lower id; length = the fewest cubes of any subset
    whose probability mass reaches `mass` (clamped), found by enumeration."""
    nc = row.shape[0]
    assert np.all(np.diff(ids) > 0) and 0 <= ids.min() and ids.max() < nc
    rest = np.setdiff1d(np.arange(nc), ids)
    for j in rest:
        for i in ids:
            assert row[i] > row[j] or (row[i] == row[j] and i < j)
    p = _softmax_lib(row)
    best = nc
    for size in range(1, nc + 1):
        if any(p[list(c)].sum() >= mass for c in itertools.combinations(range(nc), size)):
            best = size
            break
    assert len(ids) == min(max(best, k_min), k_max)


@pytest.mark.parametrize("mass", [0.05, 0.3, 0.5, 0.8, 0.95])
def test_mass_rule_matches_subset_enumeration(mass):
    rng = np.random.default_rng(int(mass * 100))
    S = 1.5 * rng.standard_normal((12, 8))
    S[4, :] = rng.standard_normal(8) * 1e-3  # a nearly flat row
    lists, lengths = vo.select_mass(S, mass, 1, 8)
    for r in range(S.shape[0]):
        assert lengths[r] == len(lists[r])
        _check_mass_list(S[r], lists[r], mass, 1, 8)
    lists, _ = vo.select_mass(S, mass, 2, 5)  # clamped
    for r in range(S.shape[0]):
        _check_mass_list(S[r], lists[r], mass, 2, 5)


def test_mass_rule_is_topk_when_clamped_to_one_length():
    rng = np.random.default_rng(5)
    S = rng.standard_normal((10, 40))
    S[:, 7] = S[:, 30]  # exact ties
    for K in (1, 4, 17, 40):
        for mass in (0.01, 0.5, 1.0):
            lists, lengths = vo.select_mass(S, mass, K, K)
            assert np.all(lengths == K)
            np.testing.assert_array_equal(np.array(lists), _rank_select(S, K))


def test_mass_rule_uniform_row_closed_form():
    nc = 40
    S = np.full((1, nc), 0.7)  # every cube has probability 1/nc
    for m in (1, 3, 10, 25, 40):
        lists, lengths = vo.select_mass(S, (m - 0.5) / nc, 1, nc)
        assert lengths[0] == m  # ceil(mass * nc)
        np.testing.assert_array_equal(lists[0], np.arange(m))  # ties: lowest ids


def test_mass_rule_monotone_nested_and_clamped():
    rng = np.random.default_rng(11)
    S = 2.0 * rng.standard_normal((6, 64))
    prev = None
    for mass in (0.1, 0.25, 0.5, 0.75, 0.9, 0.99):
        lists, lengths = vo.select_mass(S, mass, 1, 64)
        if prev is not None:
            assert np.all(lengths >= prev[1])
            for a, b in zip(prev[0], lists):
                assert set(a) <= set(b)
        prev = (lists, lengths)
    _, lengths = vo.select_mass(S, 1e-9, 3, 64)
    assert np.all(lengths == 3)  # the single largest cube already carries the mass
    _, lengths = vo.select_mass(S, 1.0, 1, 20)
    assert np.all(lengths == 20)
    with pytest.raises(ValueError):
        vo.select_mass(S, 0.0, 1, 4)
    with pytest.raises(ValueError):
        vo.select_mass(S, 0.5, 5, 4)
    with pytest.raises(ValueError):
        vo.select_mass(S, 0.5, 1, 65)


def test_exact_tie_from_copied_key_cube_goes_to_lower_index():
    T, H, W = 4, 8, 12  # 6 cubes
    inp = small(nh=1, D=8, seed=3)
    members = vo.cube_members(T, H, W)
    k = inp["k"].copy()
    k[0, members[4], 0] = k[0, members[1], 0]  # cube 4 becomes a copy of cube 1
    r = oracle.forward(inp["q"], k, inp["v"], inp["gc"], inp["gf"], (T, H, W), 1)
    S = r["S"][0, 0]
    assert np.array_equal(S[:, 1], S[:, 4])
    for row in range(6):
        order = sorted(range(6), key=lambda j: (-S[row, j], j))
        K = order.index(1) + 1  # cube 1 is the last one chosen; cube 4 ties it
        assert order[K] == 4
        sel = vo.select_topk(S[row:row + 1], K)[0]
        assert 1 in sel and 4 not in sel


# ---------------------------------------------------------------- step 4: fine
def test_fine_with_all_cubes_is_dense_attention():
    inp = small(B=1, nh=2, D=16, grid=(4, 8, 12), seed=11)
    grid = (4, 8, 12)
    r = oracle.forward(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], grid, 6)
    for h in range(2):
        q, k, v = (inp[n][0, :, h].astype(np.float64) for n in "qkv")
        np.testing.assert_allclose(r["of"][0, :, h], sdpa64(q, k, v), rtol=1e-11, atol=1e-12)
        assert np.all(r["sel"][0, h] == np.arange(6))


def _brute_force_token(q, k, v, grid, key_cubes, i, scale):
    """One query token by scalar loops: walks the grid, keeps keys whose
    (t//4, y//4, x//4) block is one of key_cubes; builds no permutation."""
    T, H, W = grid
    blocks = {((c // ((W // 4) * (H // 4))), (c // (W // 4)) % (H // 4), c % (W // 4)) for c in key_cubes}
    logits, vals = [], []
    for t in range(T):
        for y in range(H):
            for x in range(W):
                if (t // 4, y // 4, x // 4) in blocks:
                    j = (t * H + y) * W + x
                    logits.append(scale * sum(float(q[i, d]) * float(k[j, d]) for d in range(q.shape[1])))
                    vals.append(v[j])
    m = max(logits)
    w = [math.exp(l - m) for l in logits]
    z = sum(w)
    return sum(wi * vi for wi, vi in zip(w, vals)) / z


def test_fine_tiny_grid_brute_force():
    grid = (8, 8, 8)
    inp = make_inputs(1, 1, 8, grid, dtype="f32", seed=5)
    r = oracle.forward(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], grid, 2)
    q, k, v = (inp[n][0, :, 0].astype(np.float64) for n in "qkv")
    cube, _ = vo.token_cube_map(*grid)
    rng = np.random.default_rng(0)
    for i in rng.choice(512, size=24, replace=False):
        ref = _brute_force_token(q, k, v, grid, set(r["sel"][0, 0, cube[i]].tolist()), i, 1 / math.sqrt(8))
        np.testing.assert_allclose(r["of"][0, i, 0], ref, rtol=1e-12, atol=1e-12)


def test_fine_constant_values_and_key_shift():
    grid = (4, 8, 8)
    inp = small(nh=1, D=8, grid=grid, seed=9)
    v = np.tile(np.arange(8.0)[None, None, None, :], (1, 256, 1, 1))
    r = oracle.forward(inp["q"], inp["k"], v, inp["gc"], inp["gf"], grid, 2)
    np.testing.assert_allclose(r["of"][0, :, 0], v[0, :, 0], rtol=1e-13, atol=1e-13)
    r1 = oracle.forward(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], grid, 2)
    r2 = oracle.forward(inp["q"], inp["k"] + 0.7 * np.arange(8.0), inp["v"], inp["gc"], inp["gf"], grid, 2)
    np.testing.assert_array_equal(r1["sel"], r2["sel"])
    np.testing.assert_allclose(r1["o"], r2["o"], rtol=1e-10, atol=1e-11)


def test_empty_list_gives_zero_fine_output():
    grid = (4, 4, 8)
    inp = small(nh=1, D=4, grid=grid, seed=2)
    lists = [[[np.array([], dtype=np.int64), np.array([0])]]]
    r = oracle.forward_with_sets(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], grid, lists)
    members = vo.cube_members(*grid)
    assert np.all(r["of"][0, members[0], 0] == 0)
    assert np.all(np.isneginf(r["lse_f"][0, 0, members[0]]))


# ---------------------------------------------------------------- step 5: gates
def test_gate_special_cases():
    grid = (4, 8, 12)
    inp = small(seed=4, grid=grid)
    one, zero = np.ones_like(inp["gc"]), np.zeros_like(inp["gc"])
    r = oracle.forward(inp["q"], inp["k"], inp["v"], zero, one, grid, 3)
    np.testing.assert_array_equal(r["o"], r["of"])
    r = oracle.forward(inp["q"], inp["k"], inp["v"], one, zero, grid, 3)
    cube, _ = vo.token_cube_map(*grid)
    for h in range(2):
        np.testing.assert_array_equal(r["o"][0, :, h], r["oc"][0, h][cube])


# ---------------------------------------------------------------- variable lists
def test_varlen_lists_reproduce_topk_and_dense_and_order_free():
    grid = (4, 8, 12)
    inp = small(seed=6, grid=grid)
    args = (inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], grid)
    r = oracle.forward(*args, 3)
    rv = oracle.forward_with_sets(*args, oracle.lists_from_sel(r["sel"]))
    np.testing.assert_array_equal(rv["o"], r["o"])
    rng = np.random.default_rng(0)
    shuffled = [[[rng.permutation(l) for l in lh] for lh in lb] for lb in oracle.lists_from_sel(r["sel"])]
    rs = oracle.forward_with_sets(*args, shuffled)
    np.testing.assert_allclose(rs["o"], r["o"], rtol=1e-12, atol=1e-13)
    dense = oracle.forward_with_sets(*args, [[[np.arange(6)] * 6] * 2])
    for h in range(2):
        q, k, v = (inp[n][0, :, h].astype(np.float64) for n in "qkv")
        np.testing.assert_allclose(dense["of"][0, :, h], sdpa64(q, k, v), rtol=1e-11, atol=1e-12)


def test_csr_lists_roundtrip():
    offs = np.array([0, 2, 2, 5]); ids = np.array([3, 1, 0, 2, 4])
    lists = oracle.lists_from_csr(offs, ids, 1, 1, 3)
    assert [list(x) for x in lists[0][0]] == [[3, 1], [], [0, 2, 4]]


# ---------------------------------------------------------------- backward
def _loss(inp, grid, lists, dout):
    r = oracle.forward_with_sets(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], grid, lists)
    return float(np.sum(dout * r["o"]))


def _fd_check(inp, grid, K, picks, h=1e-6, rtol=1e-6, atol=1e-8):
    dout = inp["dout"].astype(np.float64)
    base = {n: inp[n].astype(np.float64) for n in ("q", "k", "v", "gc", "gf")}
    r = oracle.forward(base["q"], base["k"], base["v"], base["gc"], base["gf"], grid, K)
    lists = oracle.lists_from_sel(r["sel"])
    g = oracle.backward(base["q"], base["k"], base["v"], base["gc"], base["gf"], dout, grid, lists)
    gname = dict(q="dq", k="dk", v="dv", gc="dgc", gf="dgf")
    for name, idxs in picks.items():
        for idx in idxs:
            plus = dict(base); minus = dict(base)
            plus[name] = base[name].copy(); minus[name] = base[name].copy()
            plus[name][idx] += h; minus[name][idx] -= h
            # the selection must not move at +-h for the derivative to exist
            rp = oracle.forward(plus["q"], plus["k"], plus["v"], plus["gc"], plus["gf"], grid, K)
            assert np.array_equal(rp["sel"], r["sel"])
            fd = (_loss(plus, grid, lists, dout) - _loss(minus, grid, lists, dout)) / (2 * h)
            an = g[gname[name]][idx]
            assert abs(fd - an) <= atol + rtol * max(1.0, abs(an)), (name, idx, fd, an)
    return g, base, dout


def test_backward_finite_differences_every_element():
    grid = (4, 4, 8)
    inp = make_inputs(1, 1, 2, grid, dtype="f32", seed=21, with_dout=True)
    picks = {n: list(np.ndindex(inp[n].shape)) for n in ("q", "k", "v", "gc", "gf")}
    _fd_check(inp, grid, 1, picks)


def test_backward_finite_differences_sampled_and_invariants():
    grid = (4, 8, 12)
    inp = make_inputs(2, 2, 8, grid, dtype="f32", seed=22, with_dout=True)
    rng = np.random.default_rng(0)
    picks = {}
    for n in ("q", "k", "v", "gc", "gf"):
        shape = inp[n].shape
        flat = rng.choice(int(np.prod(shape)), size=40, replace=False)
        picks[n] = [np.unravel_index(f, shape) for f in flat]
    g, base, dout = _fd_check(inp, grid, 3, picks)
    # a common shift of all keys changes no softmax: sum of dk is zero
    np.testing.assert_allclose(g["dk"].sum(axis=1), 0.0, atol=1e-11)
    # softmax rows sum to one: sum of dv equals sum of (gc + gf) * dout
    ref = ((base["gc"] + base["gf"])[..., None] * dout).sum(axis=1)
    np.testing.assert_allclose(g["dv"].sum(axis=1), ref, rtol=1e-11, atol=1e-11)
    # closed forms for the gate gradients
    r = oracle.forward(base["q"], base["k"], base["v"], base["gc"], base["gf"], grid, 3)
    cube, _ = vo.token_cube_map(*grid)
    for b in range(2):
        for h in range(2):
            np.testing.assert_allclose(g["dgc"][b, :, h], (dout[b, :, h] * r["oc"][b, h][cube]).sum(1), rtol=1e-12)
            np.testing.assert_allclose(g["dgf"][b, :, h], (dout[b, :, h] * r["of"][b, :, h]).sum(1), rtol=1e-12)


# ---------------------------------------------------------------- sampled helper
def test_query_cube_output_matches_forward():
    grid = (4, 8, 12)
    inp = small(seed=13, grid=grid)
    r = oracle.forward(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], grid, 2)
    for (b, h, c) in [(0, 0, 0), (0, 1, 5), (0, 1, 3)]:
        rows, o, oc_row, logits = oracle.query_cube_output(
            inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], grid, b, h, c, r["sel"][b, h, c])
        np.testing.assert_allclose(o, r["o"][b, rows, h], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(logits, r["S"][b, h, c], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- pages' figures
def test_pages_sparsity_figure_at_16k_tokens():
    fig = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))
    T, H, W = fig["pretrain_grid"]
    K = fig["pretrain_topk"]
    assert T * H * W == fig["pretrain_tokens"]
    assert fig["cube"] == [4, 4, 4] and vo.CUBE_TOKENS == 64
    inp = make_inputs(1, 1, 4, (T, H, W), dtype="f32", seed=0)
    r = oracle.forward(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], (T, H, W), K)
    nc = T * H * W // 64
    kept = r["sel"].shape[-1] * 64 / (nc * 64)
    assert abs((1 - kept) - fig["sparsity"]) < 1e-12


def test_backward_sampled_matches_full_backward():
    grid = (4, 8, 12)
    inp = make_inputs(2, 2, 8, grid, dtype="f32", seed=23, with_dout=True)
    r = oracle.forward(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], grid, 3)
    lists = oracle.lists_from_sel(r["sel"])
    lists[1][0][2] = []  # an empty list
    g = oracle.backward(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], inp["dout"], grid, lists)
    members = vo.cube_members(*grid)
    for b, h in [(0, 1), (1, 0)]:
        out = oracle.backward_sampled(inp["q"], inp["k"], inp["v"], inp["gc"], inp["gf"], inp["dout"],
                                      grid, lists[b][h], b, h, [0, 2, 5], [1, 2, 4])
        for c in (0, 2, 5):
            np.testing.assert_allclose(out[("dq", c)], g["dq"][b, members[c], h], rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(out[("dgc", c)], g["dgc"][b, members[c], h], rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(out[("dgf", c)], g["dgf"][b, members[c], h], rtol=1e-11, atol=1e-12)
        for j in (1, 2, 4):
            np.testing.assert_allclose(out[("dk", j)], g["dk"][b, members[j], h], rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(out[("dv", j)], g["dv"][b, members[j], h], rtol=1e-11, atol=1e-12)
