"""fp64 CPU oracle for hierarchical video sparse attention (VSA, with the
variable-length key lists of VSA2).

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
definition that the HIP library is checked against.  Only the test suite, the
package smoke check and the benchmark's CPU-baseline leg may import it.  It
shares no code with the HIP path and imports nothing from it.

Sources (cited by page title and section):
  [VSA-abs]  "VSA: Faster Video Diffusion with Trainable Sparse Attention",
             section "Abstract (arXiv)".
  [VSA-sum]  "Faster Video Diffusion with Trainable Sparse Attention"
             (AI-extracted summary page), sections "Approach",
             "Key results", "Surprising findings", "Limitations".
  [VSA2-abs] "Improving Video Sparse Attention with Fine-grained Router and
             Sparse Rebasing", section "Abstract (arXiv)".

What is computed, per (batch, head), following [VSA-sum, Approach] and
[VSA-abs]:
  1. tokens of the T x H x W grid are grouped into 4x4x4 cubes of 64 tokens
     ([VSA-sum, Approach]; dimensions divisible by 4 per [VSA-sum,
     Limitations]);
  2. Q, K and V are mean-pooled per cube, and dense cube-to-cube attention on
     the pooled tensors gives a coarse output per cube ([VSA-sum, Approach]:
     mean pooling, coarse cube-to-cube attention, coarse context);
  3. the coarse scores of each query cube pick its top-K key cubes
     ([VSA-sum, Approach]);
  4. token-level attention runs only over the tokens of the selected cubes
     ([VSA-abs]: the fine stage attends only inside the chosen tiles);
  5. the two outputs are combined with gates ([VSA-sum, Approach]).
  Variable-length lists ([VSA2-abs]: each query may attend a variable number
  of key-value pairs) replace step 3 by caller-given cube lists.

Readings taken where the pages are silent (each one is also listed in the
design notes of the repository):
  * softmax scale s = 1/sqrt(head_dim) in both stages;
  * tokens are in raster order, flat index (t*H + y)*W + x, t slowest;
  * cubes are numbered in raster order over the (T/4, H/4, W/4) cube grid;
  * a token's slot inside its cube is ((t%4)*4 + y%4)*4 + x%4;
  * the coarse scores that rank key cubes are the coarse logits; ties go to
    the lower cube index; the selected list is reported ascending;
  * the query's own cube is not forced into its selection;
  * selection is per (batch, head);
  * gates are one scalar per (batch, token, head), broadcast over head_dim;
  * the coarse output of a cube is broadcast to its 64 tokens;
  * no gradient flows through the (piecewise constant) selection;
  * an empty key list gives a zero fine output and log-sum-exp -inf.

Arrays are float64 numpy; q, k, v, dout: [B, N, heads, D]; gates [B, N, heads].
Parity status: every function here is pinned by tests against independent
references (library dense attention, brute-force loops, closed forms,
invariants and finite differences).
"""
from __future__ import annotations

import numpy as np

CUBE = 4  # cube edge, [VSA-sum, Approach]
CUBE_TOKENS = CUBE * CUBE * CUBE


def _check_grid(T, H, W):
    if T <= 0 or H <= 0 or W <= 0 or T % CUBE or H % CUBE or W % CUBE:
        # [VSA-sum, Limitations]: latent dimensions must be divisible by 4.
        raise ValueError(f"grid {T}x{H}x{W} is not made of 4x4x4 cubes")


def token_cube_map(T, H, W):
    """Cube id and in-cube slot of every raster token ([VSA-sum, Approach]).

    Returns (cube, slot), int64 arrays of length N = T*H*W.
    """
    _check_grid(T, H, W)
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    t, y, x = t.ravel(), y.ravel(), x.ravel()
    cube = ((t // CUBE) * (H // CUBE) + y // CUBE) * (W // CUBE) + x // CUBE
    slot = ((t % CUBE) * CUBE + y % CUBE) * CUBE + x % CUBE
    return cube.astype(np.int64), slot.astype(np.int64)


def cube_members(T, H, W):
    """[Nc, 64] raster token indices of each cube, ordered by slot."""
    cube, slot = token_cube_map(T, H, W)
    nc = cube.max() + 1
    members = np.empty((nc, CUBE_TOKENS), dtype=np.int64)
    members[cube, slot] = np.arange(T * H * W)
    return members


def pool(x, T, H, W, op="mean"):
    """Mean of the 64 tokens of each cube ([VSA-sum, Approach]: mean pooling).

    op="max" takes the per-channel maximum instead, the alternative that the
    pooling ablation compares against ([VSA-sum, Surprising findings]: mean
    pooling did better than max and convolutional pooling).
    x: [N, D] for one (batch, head).  Returns [Nc, D].
    """
    members = cube_members(T, H, W)
    if op == "mean":
        return x[members].mean(axis=1)
    if op == "max":
        return x[members].max(axis=1)
    raise ValueError(f"unknown pooling {op!r}")


def cube_attention_mass(q, k, grid, b, h, c, scale=None):
    """Share of the dense attention of query cube c that lands on each key
    cube, for one (batch b, head h): every query token of cube c attends to
    all N keys with a softmax of s q.k; its weights are summed over the 64
    tokens of each key cube and averaged over the cube's 64 queries.  The
    key cubes with the most mass are the "critical" ones that the coarse
    stage tries to find ([VSA-abs]: the attention mass concentrates on a
    small subset of positions; [VSA-sum, Key results] lists critical-token
    prediction accuracy among the metrics).  Returns [Nc], summing to 1.
    """
    T, H, W = grid
    members = cube_members(T, H, W)
    D = q.shape[-1]
    s = 1.0 / np.sqrt(D) if scale is None else scale
    Q = _as64(q[b, members[c], h])  # [64, D]
    K = _as64(k[b, :, h])           # [N, D]
    Pm, _ = _softmax_rows(s * (Q @ K.T))
    return Pm[:, members].sum(axis=2).mean(axis=0)


def _softmax_rows(logits):
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    z = e.sum(axis=1, keepdims=True)
    return e / z, (m + np.log(z))[:, 0]


def coarse_attention(qc, kc, vc, scale):
    """Dense cube-to-cube attention on pooled tensors ([VSA-sum, Approach]).

    Returns (Oc [Nc, D], logits S [Nc, Nc], lse [Nc]).  Every key cube is
    visible to every query cube, including its own.
    """
    S = scale * (qc @ kc.T)
    P, lse = _softmax_rows(S)
    return P @ vc, S, lse


def select_topk(S, topk):
    """Top-K key cubes per query cube by coarse logit ([VSA-sum, Approach]).

    Ranks by (logit descending, cube index ascending) and reports each row's
    chosen ids in ascending order.  Returns int64 [Nc, topk].
    """
    nc = S.shape[1]
    if not 1 <= topk <= nc:
        raise ValueError(f"topk={topk} outside [1, {nc}]")
    idx = np.arange(nc)
    sel = np.empty((S.shape[0], topk), dtype=np.int64)
    for r in range(S.shape[0]):
        order = np.lexsort((idx, -S[r]))  # primary key: -S, then index
        sel[r] = np.sort(order[:topk])
    return sel


def select_mass(S, mass, k_min, k_max):
    """Stand-in variable-length selection: key-cube lists of varying length
    per query cube, as [VSA2-abs] lets each query attend a variable number
    of key-value pairs.  The pages do not define how VSA2 picks them (its
    router is not given), so this rule is an assumption of this library, not
    the method: for each query cube, rank the key cubes as select_topk does
    (coarse logit descending, cube index ascending) and take the shortest
    prefix of that ranking whose coarse softmax probability mass reaches
    `mass` ([VSA-sum, Approach]: the coarse scores mark the critical
    cubes); clamp its length to [k_min, k_max].

    Returns (lists, lengths): a list of ascending int64 arrays, one per row
    of S, and their lengths.  0 < mass <= 1, 1 <= k_min <= k_max <= Nc.
    """
    nc = S.shape[1]
    if not (0.0 < mass <= 1.0 and 1 <= k_min <= k_max <= nc):
        raise ValueError(f"mass={mass}, k_min={k_min}, k_max={k_max} out of range for Nc={nc}")
    P, _ = _softmax_rows(S)
    idx = np.arange(nc)
    lists, lengths = [], np.empty(S.shape[0], dtype=np.int64)
    for r in range(S.shape[0]):
        order = np.lexsort((idx, -S[r]))
        reached = np.nonzero(np.cumsum(P[r, order]) >= mass)[0]
        n = int(reached[0]) + 1 if reached.size else nc
        n = min(max(n, k_min), k_max)
        lists.append(np.sort(order[:n]))
        lengths[r] = n
    return lists, lengths


def fine_attention(q, k, v, key_lists, T, H, W, scale):
    """Token-level softmax attention restricted to the selected cubes
    ([VSA-abs]: the fine stage attends only inside the selected tiles).

    q, k, v: [N, D] of one (batch, head); key_lists[c] = key cube ids of
    query cube c.  Returns (O_fine [N, D], lse [N]) in raster token order.
    """
    members = cube_members(T, H, W)
    N, D = q.shape
    out = np.zeros((N, D))
    lse = np.full(N, -np.inf)
    for c in range(members.shape[0]):
        ids = np.asarray(key_lists[c], dtype=np.int64)
        if ids.size == 0:
            continue
        rows = members[c]
        keys = members[ids].ravel()
        P, l = _softmax_rows(scale * (q[rows] @ k[keys].T))
        out[rows] = P @ v[keys]
        lse[rows] = l
    return out, lse


def _forward_bh(q, k, v, gc, gf, grid, key_lists, topk, scale):
    T, H, W = grid
    cube, _ = token_cube_map(T, H, W)
    qc, kc, vc = pool(q, T, H, W), pool(k, T, H, W), pool(v, T, H, W)
    oc, S, lse_c = coarse_attention(qc, kc, vc, scale)
    sel = None
    if key_lists is None:
        sel = select_topk(S, topk)
        key_lists = list(sel)
    of, lse_f = fine_attention(q, k, v, key_lists, T, H, W, scale)
    # [VSA-sum, Approach]: gated combination of coarse and fine outputs.
    o = gc[:, None] * oc[cube] + gf[:, None] * of
    return dict(o=o, sel=sel, oc=oc, S=S, lse_c=lse_c, of=of, lse_f=lse_f,
                qc=qc, kc=kc, vc=vc)


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def forward(q, k, v, gc, gf, grid, topk, scale=None, key_lists=None):
    """Full forward.  If key_lists is given (indexable [b][h][c]) it replaces
    the top-K selection (the variable-length entry point, [VSA2-abs]).

    Returns a dict: o [B,N,nh,D]; sel [B,nh,Nc,topk] (None with key_lists);
    oc [B,nh,Nc,D]; S [B,nh,Nc,Nc]; lse_c [B,nh,Nc]; of [B,N,nh,D];
    lse_f [B,nh,N].
    """
    q, k, v, gc, gf = map(_as64, (q, k, v, gc, gf))
    B, N, nh, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    res = dict(o=np.zeros_like(q), of=np.zeros_like(q), lse_f=np.zeros((B, nh, N)),
               sel=None, oc=[], S=[], lse_c=[])
    sels = []
    for b in range(B):
        for h in range(nh):
            lists = None if key_lists is None else key_lists[b][h]
            r = _forward_bh(q[b, :, h], k[b, :, h], v[b, :, h], gc[b, :, h], gf[b, :, h],
                            grid, lists, topk, scale)
            res["o"][b, :, h] = r["o"]
            res["of"][b, :, h] = r["of"]
            res["lse_f"][b, h] = r["lse_f"]
            res["oc"].append(r["oc"])
            res["S"].append(r["S"])
            res["lse_c"].append(r["lse_c"])
            sels.append(r["sel"])
    nc = res["oc"][0].shape[0]
    res["oc"] = np.stack(res["oc"]).reshape(B, nh, nc, D)
    res["S"] = np.stack(res["S"]).reshape(B, nh, nc, nc)
    res["lse_c"] = np.stack(res["lse_c"]).reshape(B, nh, nc)
    if key_lists is None:
        res["sel"] = np.stack(sels).reshape(B, nh, nc, topk)
    return res


def forward_with_sets(q, k, v, gc, gf, grid, key_lists, scale=None):
    """forward() with the selection given, e.g. the GPU's own index set or a
    variable-length list per query cube ([VSA2-abs])."""
    return forward(q, k, v, gc, gf, grid, topk=None, scale=scale, key_lists=key_lists)


def lists_from_csr(offsets, ids, B, nh, nc):
    """Per-(b, h, c) key-cube lists from CSR offsets/ids ordered (b, h, c)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    ids = np.asarray(ids, dtype=np.int64)
    lists = [[[None] * nc for _ in range(nh)] for _ in range(B)]
    for b in range(B):
        for h in range(nh):
            for c in range(nc):
                r = (b * nh + h) * nc + c
                lists[b][h][c] = ids[offsets[r]:offsets[r + 1]]
    return lists


def lists_from_sel(sel):
    """Per-(b, h, c) lists from a [B, nh, Nc, K] selection array."""
    sel = np.asarray(sel)
    return [[list(sel[b, h]) for h in range(sel.shape[1])] for b in range(sel.shape[0])]


def backward(q, k, v, gc, gf, dout, grid, key_lists, scale=None):
    """Gradients of sum(dout * o) with the selection held fixed
    ([VSA-abs]: the operator trains end-to-end; no gradient is defined
    through the discrete top-K choice, so the coarse path carries the
    gradient to the pooled tensors).

    key_lists: [b][h][c] key cube ids (the forward's selection).
    Returns dict dq, dk, dv [B,N,nh,D], dgc, dgf [B,N,nh].
    """
    q, k, v, gc, gf, dout = map(_as64, (q, k, v, gc, gf, dout))
    B, N, nh, D = q.shape
    T, H, W = grid
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    members = cube_members(T, H, W)
    cube, _ = token_cube_map(T, H, W)
    nc = members.shape[0]
    g = dict(dq=np.zeros_like(q), dk=np.zeros_like(q), dv=np.zeros_like(q),
             dgc=np.zeros_like(gc), dgf=np.zeros_like(gf))
    for b in range(B):
        for h in range(nh):
            qb, kb, vb = q[b, :, h], k[b, :, h], v[b, :, h]
            G = dout[b, :, h]
            r = _forward_bh(qb, kb, vb, gc[b, :, h], gf[b, :, h], grid,
                            key_lists[b][h], None, scale)
            dq, dk, dv = np.zeros((N, D)), np.zeros((N, D)), np.zeros((N, D))
            # o = gc * Oc[cube] + gf * Of
            g["dgc"][b, :, h] = np.sum(G * r["oc"][cube], axis=1)
            g["dgf"][b, :, h] = np.sum(G * r["of"], axis=1)
            # fine stage: softmax attention over the selected tokens
            dOf = gf[b, :, h][:, None] * G
            for c in range(nc):
                ids = np.asarray(key_lists[b][h][c], dtype=np.int64)
                if ids.size == 0:
                    continue
                rows = members[c]
                keys = members[ids].ravel()
                P = np.exp(scale * (qb[rows] @ kb[keys].T) - r["lse_f"][rows][:, None])
                delta = np.sum(dOf[rows] * r["of"][rows], axis=1)
                dP = dOf[rows] @ vb[keys].T
                dS = P * (dP - delta[:, None])
                dq[rows] += scale * (dS @ kb[keys])
                np.add.at(dk, keys, scale * (dS.T @ qb[rows]))
                np.add.at(dv, keys, P.T @ dOf[rows])
            # coarse stage: dense attention on pooled tensors
            dOc = np.zeros((nc, D))
            np.add.at(dOc, cube, gc[b, :, h][:, None] * G)
            Pc = np.exp(r["S"] - r["lse_c"][:, None])
            dVc = Pc.T @ dOc
            dPc = dOc @ r["vc"].T
            dSc = Pc * (dPc - np.sum(dOc * r["oc"], axis=1)[:, None])
            dQc = scale * (dSc @ r["kc"])
            dKc = scale * (dSc.T @ r["qc"])
            # adjoint of the 64-token mean
            dq += dQc[cube] / CUBE_TOKENS
            dk += dKc[cube] / CUBE_TOKENS
            dv += dVc[cube] / CUBE_TOKENS
            g["dq"][b, :, h], g["dk"][b, :, h], g["dv"][b, :, h] = dq, dk, dv
    return g


def query_cube_output(q, k, v, gc, gf, grid, b, h, c, key_ids, scale=None):
    """Output rows of one query cube (b, h, c) given its key-cube list, for
    sampled checks at sizes where the full forward is too slow.  The coarse
    output is recomputed from the pooled tensors of head (b, h).

    Returns (raster token indices [64], o [64, D], oc_row [D], logits [Nc]).
    """
    T, H, W = grid
    qb = _as64(q[b, :, h]); kb = _as64(k[b, :, h]); vb = _as64(v[b, :, h])
    D = qb.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    members = cube_members(T, H, W)
    qc_row = qb[members[c]].mean(axis=0)
    kc = pool(kb, T, H, W)
    vc = pool(vb, T, H, W)
    logits = scale * (kc @ qc_row)
    p = np.exp(logits - logits.max())
    oc_row = (p / p.sum()) @ vc
    rows = members[c]
    ids = np.asarray(key_ids, dtype=np.int64)
    if ids.size:
        keys = members[ids].ravel()
        P, _ = _softmax_rows(scale * (qb[rows] @ kb[keys].T))
        of = P @ vb[keys]
    else:
        of = np.zeros((64, D))
    o = _as64(gc[b, rows, h])[:, None] * oc_row[None, :] + _as64(gf[b, rows, h])[:, None] * of
    return rows, o, oc_row, logits


def backward_sampled(q, k, v, gc, gf, dout, grid, key_lists_bh, b, h, query_cubes, key_cubes,
                     scale=None):
    """Gradients of sum(dout * o) for one (batch, head), restricted to a few
    cubes, with the same formulas as backward(): dq, dg_c and dg_f of the
    tokens of `query_cubes`; dk and dv of the tokens of `key_cubes`.  Used
    for sampled checks where the full backward is too slow.

    key_lists_bh[c]: key cube ids of query cube c for this (b, h).
    Returns dict: for each query cube c, ("dq", c) -> [64, D] and
    ("dgc", c), ("dgf", c) -> [64]; for each key cube j, ("dk", j), ("dv", j)
    -> [64, D]; rows ordered as cube_members(...)[cube].
    """
    T, H, W = grid
    qb = _as64(q[b, :, h]); kb = _as64(k[b, :, h]); vb = _as64(v[b, :, h])
    G = _as64(dout[b, :, h]); gcb = _as64(gc[b, :, h]); gfb = _as64(gf[b, :, h])
    D = qb.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    members = cube_members(T, H, W)
    cube, _ = token_cube_map(T, H, W)
    nc = members.shape[0]
    qc, kc, vc = pool(qb, T, H, W), pool(kb, T, H, W), pool(vb, T, H, W)
    oc, S, lse_c = coarse_attention(qc, kc, vc, scale)
    # coarse backward (whole head; it is small)
    dOc = np.zeros((nc, D))
    np.add.at(dOc, cube, gcb[:, None] * G)
    Pc = np.exp(S - lse_c[:, None])
    dVc = Pc.T @ dOc
    dSc = Pc * (dOc @ vc.T - np.sum(dOc * oc, axis=1)[:, None])
    dQc = scale * (dSc @ kc)
    dKc = scale * (dSc.T @ qc)
    key_set = set(int(j) for j in key_cubes)
    needed = set(int(c) for c in query_cubes)
    for c in range(nc):
        if key_set.intersection(int(j) for j in key_lists_bh[c]):
            needed.add(c)
    out = {}
    for j in key_set:
        out[("dk", j)] = dKc[j][None, :].repeat(64, 0) / CUBE_TOKENS
        out[("dv", j)] = dVc[j][None, :].repeat(64, 0) / CUBE_TOKENS
    for c in sorted(needed):
        rows = members[c]
        ids = np.asarray(key_lists_bh[c], dtype=np.int64)
        if c in query_cubes:
            out[("dq", c)] = dQc[c][None, :].repeat(64, 0) / CUBE_TOKENS
        if ids.size == 0:
            if c in query_cubes:
                out[("dgc", c)] = np.sum(G[rows] * oc[c], axis=1)
                out[("dgf", c)] = np.zeros(64)
            continue
        keys = members[ids].ravel()
        P, _ = _softmax_rows(scale * (qb[rows] @ kb[keys].T))
        of = P @ vb[keys]
        dOf = gfb[rows][:, None] * G[rows]
        delta = np.sum(dOf * of, axis=1)
        dS = P * (dOf @ vb[keys].T - delta[:, None])
        if c in query_cubes:
            out[("dq", c)] = out[("dq", c)] + scale * (dS @ kb[keys])
            out[("dgc", c)] = np.sum(G[rows] * oc[c], axis=1)
            out[("dgf", c)] = np.sum(G[rows] * of, axis=1)
        for pos, j in enumerate(ids):
            j = int(j)
            if j in key_set:
                sl = slice(64 * pos, 64 * pos + 64)
                out[("dk", j)] = out[("dk", j)] + scale * (dS[:, sl].T @ qb[rows])
                out[("dv", j)] = out[("dv", j)] + P[:, sl].T @ dOf
    return out
