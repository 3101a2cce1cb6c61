"""PyTorch-facing binding of libvsa.so.

Argument marshalling only: shape/dtype checks, output and workspace
allocation through torch's caching allocator, raw device pointers and the
current HIP stream handed to the C entry points of include/vsa.h.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback path.  Tensors use raster token order:
q, k, v, out: [B, N, heads, D]; gates: [B, N, heads]; N = T*H*W.
"""
from __future__ import annotations

import contextlib

import torch

from . import _lib

_DT = {torch.float32: _lib.VSA_F32, torch.bfloat16: _lib.VSA_BF16}


@contextlib.contextmanager
def _on(t):
    """Runs the enclosed library call with t's GPU as the current device and
    yields that device's current stream: the kernels launch where the
    tensors live, whichever device the caller has current."""
    with torch.cuda.device(t.device):
        yield torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check_inputs(q, k, v, gate_c, gate_f, grid):
    if q.dtype not in _DT:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v), ("gate_c", gate_c), ("gate_f", gate_f)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != q.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {q.dtype}")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, N, heads, D] shape")
    B, N, nh, D = q.shape
    T, H, W = grid
    if T * H * W != N:
        raise ValueError(f"grid {grid} has {T * H * W} tokens, tensors have {N}")
    if gate_c.shape != (B, N, nh) or gate_f.shape != (B, N, nh):
        raise ValueError("gates must be [B, N, heads]")
    return B, N, nh, D, T, H, W, _DT[q.dtype]


def _need(t, name, dtype, shape=None, numel=None, min_numel=None, device=None):
    """A tensor handed to the C ABI as a raw pointer: on the GPU (on
    `device` when given), dense, of the element type (and shape or size) the
    call assumes."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs at least {min_numel}")


def _check_qkv(q, k, v, grid):
    if q.dtype not in _DT:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype, shape=q.shape, device=q.device)
    if q.dim() != 4 or q.shape[1] != grid[0] * grid[1] * grid[2]:
        raise ValueError(f"q must be [B, N, heads, D] with N = {grid[0] * grid[1] * grid[2]}")


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def saved_bytes(B, heads, D, grid, dtype=torch.bfloat16):
    if dtype not in _DT:
        raise TypeError(f"unsupported dtype {dtype}")
    return _lib.load().vsa_saved_bytes(B, heads, D, *grid, _DT[dtype])


def _out(out, q):
    if out is None:
        return torch.empty_like(q)
    _need(out, "out", q.dtype, shape=q.shape, device=q.device)
    return out


def vsa_forward(q, k, v, gate_c, gate_f, grid, topk, save=False, out=None):
    """Returns (out, sel_idx [B, heads, Nc, topk] int32, saved or None).
    `out` (optional) is the tensor to write the result into."""
    lib = _lib.load()
    B, N, nh, D, T, H, W, dt = _check_inputs(q, k, v, gate_c, gate_f, grid)
    nc = N // 64
    out = _out(out, q)
    sel = torch.empty((B, nh, nc, topk), dtype=torch.int32, device=q.device)
    saved = _workspace(lib.vsa_saved_bytes(B, nh, D, T, H, W, dt), q.device) if save else None
    wsb = lib.vsa_forward_workspace_bytes(B, nh, D, T, H, W, dt)
    ws = _workspace(wsb, q.device)
    with _on(q) as stream:
        st = lib.vsa_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(gate_c), _ptr(gate_f),
                             B, nh, D, T, H, W, topk, dt, _ptr(out), _ptr(sel), _ptr(saved),
                             _ptr(ws), wsb, stream)
    _lib.check("vsa_forward", st)
    return out, sel, saved


def validate_lists(kv_ids, n_rows, n_cubes, kv_offsets=None, topk=0):
    """Checks key lists on the GPU (include/vsa.h, vsa_validate_lists) and
    returns (offset_faults, bad_lists); (0, 0) means well formed.  Reading
    the answer waits for the current stream."""
    lib = _lib.load()
    _need(kv_ids, "kv_ids", torch.int32, device=kv_ids.device)
    if kv_offsets is not None:
        _need(kv_offsets, "kv_offsets", torch.int32, numel=n_rows + 1, device=kv_ids.device)
    result = torch.empty(2, dtype=torch.int32, device=kv_ids.device)
    with _on(kv_ids) as stream:
        st = lib.vsa_validate_lists(_ptr(kv_offsets), _ptr(kv_ids), int(kv_ids.numel()), int(topk),
                                    int(n_rows), int(n_cubes), _ptr(result), stream)
    _lib.check("vsa_validate_lists", st)
    faults, bad = (int(x) for x in result.tolist())
    return faults, bad


def _require_valid(kv_ids, n_rows, n_cubes, kv_offsets=None, topk=0):
    faults, bad = validate_lists(kv_ids, n_rows, n_cubes, kv_offsets=kv_offsets, topk=topk)
    if faults or bad:
        raise ValueError(f"malformed key lists: {faults} offset fault(s), {bad} list(s) with an id "
                         f"outside [0, {n_cubes}) or repeated")


def _check_lists(kv_offsets, kv_ids, B, nh, nc):
    for name, t in (("kv_offsets", kv_offsets), ("kv_ids", kv_ids)):
        if not t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 GPU tensor")
    if kv_ids.device != kv_offsets.device:
        raise ValueError("kv_offsets and kv_ids must be on one device")
    if kv_offsets.shape != (B * nh * nc + 1,):
        raise ValueError("kv_offsets must have B*heads*Nc + 1 entries")


def block_sparse_attn_varlen(q, k, v, gate_c, gate_f, grid, kv_offsets, kv_ids, save=False,
                             out=None, validate=True):
    """Variable-length key-cube lists (CSR over (b, h, query cube)).
    Returns (out, saved or None).  With validate (the default) the lists are
    checked on the GPU first and a ValueError names what is wrong; that
    check waits for the stream, so hot loops with known-good lists pass
    validate=False."""
    lib = _lib.load()
    B, N, nh, D, T, H, W, dt = _check_inputs(q, k, v, gate_c, gate_f, grid)
    nc = N // 64
    _check_lists(kv_offsets, kv_ids, B, nh, nc)
    if validate:
        _require_valid(kv_ids, B * nh * nc, nc, kv_offsets=kv_offsets)
    out = _out(out, q)
    saved = _workspace(lib.vsa_saved_bytes(B, nh, D, T, H, W, dt), q.device) if save else None
    wsb = lib.vsa_forward_workspace_bytes(B, nh, D, T, H, W, dt)
    ws = _workspace(wsb, q.device)
    with _on(q) as stream:
        st = lib.block_sparse_attn_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(gate_c), _ptr(gate_f),
                                          B, nh, D, T, H, W, _ptr(kv_offsets), _ptr(kv_ids),
                                          int(kv_ids.numel()), dt, _ptr(out), _ptr(saved),
                                          _ptr(ws), wsb, stream)
    _lib.check("block_sparse_attn_varlen", st)
    return out, saved


def vsa_forward_mass(q, k, v, gate_c, gate_f, grid, mass, k_min, k_max, save=False, trim=True):
    """Forward with the stand-in variable-length rule of include/vsa.h (per
    query cube, the shortest logit-ranked prefix reaching `mass` of the
    coarse probability, length clamped to [k_min, k_max]).
    Returns (out, kv_offsets, kv_ids, saved or None).  With trim, kv_ids is
    cut to its kv_offsets[-1] entries, which reads that count back to the
    host (a synchronisation of the current stream); without, it keeps its
    B*heads*Nc*k_max capacity and nothing waits."""
    lib = _lib.load()
    B, N, nh, D, T, H, W, dt = _check_inputs(q, k, v, gate_c, gate_f, grid)
    nc = N // 64
    out = torch.empty_like(q)
    offs = torch.empty(B * nh * nc + 1, dtype=torch.int32, device=q.device)
    ids = torch.empty(B * nh * nc * max(int(k_max), 1), dtype=torch.int32, device=q.device)
    saved = _workspace(lib.vsa_saved_bytes(B, nh, D, T, H, W, dt), q.device) if save else None
    wsb = lib.vsa_forward_mass_workspace_bytes(B, nh, D, T, H, W, dt, int(k_max))
    ws = _workspace(wsb, q.device)
    with _on(q) as stream:
        st = lib.vsa_forward_mass(_ptr(q), _ptr(k), _ptr(v), _ptr(gate_c), _ptr(gate_f),
                                  B, nh, D, T, H, W, float(mass), int(k_min), int(k_max), dt,
                                  _ptr(out), _ptr(offs), _ptr(ids), _ptr(saved), _ptr(ws), wsb, stream)
    _lib.check("vsa_forward_mass", st)
    return out, offs, ids[:int(offs[-1].item())] if trim else ids, saved


def vsa_backward(q, k, v, gate_c, gate_f, dout, sel, saved, grid, validate=False):
    """Gradients of sum(dout * out) for a forward run with save=True.
    Returns (dq, dk, dv, dgate_c, dgate_f); gate gradients are fp32.
    validate checks a caller-made sel first (vsa_forward's own needs none)."""
    lib = _lib.load()
    B, N, nh, D, T, H, W, dt = _check_inputs(q, k, v, gate_c, gate_f, grid)
    _need(dout, "dout", q.dtype, shape=q.shape, device=q.device)
    nc = N // 64
    if sel.dim() != 4 or tuple(sel.shape[:3]) != (B, nh, nc):
        raise ValueError("sel must be [B, heads, Nc, topk]")
    _need(sel, "sel", torch.int32, device=q.device)
    if validate:
        _require_valid(sel, B * nh * nc, nc, topk=sel.shape[-1])
    _need(saved, "saved", torch.uint8, min_numel=int(lib.vsa_saved_bytes(B, nh, D, T, H, W, dt)))
    topk = sel.shape[-1]
    grads = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
             torch.empty(gate_c.shape, dtype=torch.float32, device=q.device),
             torch.empty(gate_f.shape, dtype=torch.float32, device=q.device)]
    wsb = lib.vsa_backward_workspace_bytes(B, nh, D, T, H, W, dt, int(sel.numel()))
    ws = _workspace(wsb, q.device)
    with _on(q) as stream:
        st = lib.vsa_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(gate_c), _ptr(gate_f), _ptr(dout),
                              _ptr(sel), _ptr(saved), B, nh, D, T, H, W, topk, dt,
                              *[_ptr(g) for g in grads], _ptr(ws), wsb, stream)
    _lib.check("vsa_backward", st)
    return tuple(grads)


def block_sparse_attn_varlen_backward(q, k, v, gate_c, gate_f, dout, kv_offsets, kv_ids, saved, grid,
                                      validate=True):
    """Gradients for a block_sparse_attn_varlen forward run with save=True
    and the same lists (checked first unless validate is False)."""
    lib = _lib.load()
    B, N, nh, D, T, H, W, dt = _check_inputs(q, k, v, gate_c, gate_f, grid)
    _check_lists(kv_offsets, kv_ids, B, nh, N // 64)
    if validate:
        _require_valid(kv_ids, B * nh * (N // 64), N // 64, kv_offsets=kv_offsets)
    _need(dout, "dout", q.dtype, shape=q.shape, device=q.device)
    _need(saved, "saved", torch.uint8, min_numel=int(lib.vsa_saved_bytes(B, nh, D, T, H, W, dt)))
    grads = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
             torch.empty(gate_c.shape, dtype=torch.float32, device=q.device),
             torch.empty(gate_f.shape, dtype=torch.float32, device=q.device)]
    n = int(kv_ids.numel())
    wsb = lib.vsa_backward_workspace_bytes(B, nh, D, T, H, W, dt, n)
    ws = _workspace(wsb, q.device)
    with _on(q) as stream:
        st = lib.block_sparse_attn_varlen_backward(
            _ptr(q), _ptr(k), _ptr(v), _ptr(gate_c), _ptr(gate_f), _ptr(dout),
            _ptr(kv_offsets), _ptr(kv_ids), n, _ptr(saved), B, nh, D, T, H, W, dt,
            *[_ptr(g) for g in grads], _ptr(ws), wsb, stream)
    _lib.check("block_sparse_attn_varlen_backward", st)
    return tuple(grads)


# ------------------------------------------------------------ stage calls
def _wants_grad(*ts):
    return torch.is_grad_enabled() and any(t.requires_grad for t in ts)


class _VSAFunction(torch.autograd.Function):
    """vsa_forward with its saved state, and vsa_backward as the gradient."""

    @staticmethod
    def forward(ctx, q, k, v, gate_c, gate_f, grid, topk):
        out, sel, saved = vsa_forward(q, k, v, gate_c, gate_f, grid, topk, save=True)
        ctx.save_for_backward(q, k, v, gate_c, gate_f, sel, saved)
        ctx.grid = tuple(grid)
        ctx.mark_non_differentiable(sel)
        return out, sel

    @staticmethod
    def backward(ctx, dout, _dsel):
        q, k, v, gc, gf, sel, saved = ctx.saved_tensors
        dq, dk, dv, dgc, dgf = vsa_backward(q, k, v, gc, gf, dout.contiguous(), sel, saved, ctx.grid)
        return dq, dk, dv, dgc.to(gc.dtype), dgf.to(gf.dtype), None, None


def vsa_attention(q, k, v, gate_c, gate_f, grid, topk):
    """The operator as one differentiable call: returns (out, sel_idx).
    When autograd records it, the forward keeps its saved state and the
    backward runs vsa_backward; otherwise it is vsa_forward without saved
    state.  No gradient flows through the selection.  Gate gradients come
    back in the gates' dtype (autograd wants the input's dtype), i.e. the
    fp32 gradients of vsa_backward rounded once."""
    if _wants_grad(q, k, v, gate_c, gate_f):
        return _VSAFunction.apply(q, k, v, gate_c, gate_f, tuple(grid), topk)
    out, sel, _ = vsa_forward(q, k, v, gate_c, gate_f, grid, topk)
    return out, sel


class _VarlenFunction(torch.autograd.Function):
    """block_sparse_attn_varlen with its saved state, and the varlen
    backward as the gradient (the lists were checked by the forward call
    or vouched for by the caller)."""

    @staticmethod
    def forward(ctx, q, k, v, gate_c, gate_f, grid, kv_offsets, kv_ids, validate):
        out, saved = block_sparse_attn_varlen(q, k, v, gate_c, gate_f, grid, kv_offsets, kv_ids,
                                              save=True, validate=validate)
        ctx.save_for_backward(q, k, v, gate_c, gate_f, kv_offsets, kv_ids, saved)
        ctx.grid = tuple(grid)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, gc, gf, offs, ids, saved = ctx.saved_tensors
        dq, dk, dv, dgc, dgf = block_sparse_attn_varlen_backward(
            q, k, v, gc, gf, dout.contiguous(), offs, ids, saved, ctx.grid, validate=False)
        return dq, dk, dv, dgc.to(gc.dtype), dgf.to(gf.dtype), None, None, None, None


def block_sparse_attn_varlen_attention(q, k, v, gate_c, gate_f, grid, kv_offsets, kv_ids,
                                       validate=True):
    """Differentiable form of block_sparse_attn_varlen (same lists, same
    validate switch); gate gradients as in vsa_attention.  Returns out."""
    if _wants_grad(q, k, v, gate_c, gate_f):
        return _VarlenFunction.apply(q, k, v, gate_c, gate_f, tuple(grid), kv_offsets, kv_ids, validate)
    return block_sparse_attn_varlen(q, k, v, gate_c, gate_f, grid, kv_offsets, kv_ids,
                                    validate=validate)[0]


def vsa_cube_permute_pool(q, k, v, grid, with_q_tiles=True):
    """Returns (qp, kp, vp, qc, kc, vc) in the library's cube-major layouts
    (qp is None when with_q_tiles is False, as in the forward)."""
    lib = _lib.load()
    _check_qkv(q, k, v, grid)
    B, N, nh, D = q.shape
    dt = _DT[q.dtype]
    nc = N // 64
    qp = torch.empty((B, nh, nc, 64, D), dtype=q.dtype, device=q.device) if with_q_tiles else None
    kp = torch.empty((B, nh, nc, 64, D), dtype=q.dtype, device=q.device)
    vp = torch.empty((B, nh, nc, 64, D), dtype=q.dtype, device=q.device)
    pooled = [torch.empty((B, nh, nc, D), dtype=torch.float32, device=q.device) for _ in range(3)]
    with _on(q) as stream:
        st = lib.vsa_cube_permute_pool(_ptr(q), _ptr(k), _ptr(v), B, nh, D, *grid, dt,
                                       _ptr(qp), _ptr(kp), _ptr(vp), *[_ptr(p) for p in pooled], stream)
    _lib.check("vsa_cube_permute_pool", st)
    return (qp, kp, vp, *pooled)


def vsa_cube_max_pool(q, k, v, grid):
    """Per-channel maximum of each cube's 64 tokens of q, k, v (the pooling
    ablation).  Returns fp32 (qc, kc, vc) [B, heads, Nc, D]."""
    lib = _lib.load()
    _check_qkv(q, k, v, grid)
    B, N, nh, D = q.shape
    T, H, W = grid
    nc = N // 64
    pooled = [torch.empty((B, nh, nc, D), dtype=torch.float32, device=q.device) for _ in range(3)]
    with _on(q) as stream:
        st = lib.vsa_cube_max_pool(_ptr(q), _ptr(k), _ptr(v), B, nh, D, T, H, W, _DT[q.dtype],
                                   *[_ptr(t) for t in pooled], stream)
    _lib.check("vsa_cube_max_pool", st)
    return tuple(pooled)


def vsa_coarse_topk(qc, kc, vc, topk, input_dtype=torch.float32):
    """Returns (oc, lse_c, sel or None) for fp32 pooled [B, heads, Nc, D].
    input_dtype, the element type of the attention inputs, sets the product
    precision: fp32 products for torch.float32, bf16 x 3 for torch.bfloat16
    (as the forward does for such inputs)."""
    lib = _lib.load()
    for name, t in (("qc", qc), ("kc", kc), ("vc", vc)):
        _need(t, name, torch.float32, shape=qc.shape, device=qc.device)
    B, nh, nc, D = qc.shape
    oc = torch.empty_like(qc)
    lse = torch.empty((B, nh, nc), dtype=torch.float32, device=qc.device)
    sel = torch.empty((B, nh, nc, topk), dtype=torch.int32, device=qc.device) if topk > 0 else None
    with _on(qc) as stream:
        st = lib.vsa_coarse_topk(_ptr(qc), _ptr(kc), _ptr(vc), B, nh, D, nc, topk,
                                 _DT[input_dtype], _ptr(oc), _ptr(lse), _ptr(sel), stream)
    _lib.check("vsa_coarse_topk", st)
    return oc, lse, sel


def vsa_coarse_select_mass(qc, kc, vc, mass, k_min, k_max, input_dtype=torch.float32):
    """Coarse stage with the stand-in variable-length rule.  Returns (oc,
    lse_c, counts [B, heads, Nc], ids [B, heads, Nc, k_max]); row r's list
    is ids[..., :counts[r]] (ascending)."""
    lib = _lib.load()
    for name, t in (("qc", qc), ("kc", kc), ("vc", vc)):
        _need(t, name, torch.float32, shape=qc.shape, device=qc.device)
    B, nh, nc, D = qc.shape
    oc = torch.empty_like(qc)
    lse = torch.empty((B, nh, nc), dtype=torch.float32, device=qc.device)
    counts = torch.empty((B, nh, nc), dtype=torch.int32, device=qc.device)
    ids = torch.zeros((B, nh, nc, max(int(k_max), 1)), dtype=torch.int32, device=qc.device)
    with _on(qc) as stream:
        st = lib.vsa_coarse_select_mass(_ptr(qc), _ptr(kc), _ptr(vc), B, nh, D, nc, float(mass),
                                        int(k_min), int(k_max), _DT[input_dtype], _ptr(oc), _ptr(lse),
                                        _ptr(counts), _ptr(ids), stream)
    _lib.check("vsa_coarse_select_mass", st)
    return oc, lse, counts, ids


def pack_lists(counts, ids_padded):
    """Padded lists -> CSR (kv_offsets [n_rows + 1], kv_ids with capacity
    n_rows * k_max, of which kv_offsets[-1] entries are written)."""
    lib = _lib.load()
    k_max = ids_padded.shape[-1]
    n_rows = counts.numel()
    _need(counts, "counts", torch.int32, device=counts.device)
    _need(ids_padded, "ids_padded", torch.int32, numel=n_rows * k_max, device=counts.device)
    offs = torch.empty(n_rows + 1, dtype=torch.int32, device=counts.device)
    ids = torch.empty(max(n_rows * k_max, 1), dtype=torch.int32, device=counts.device)
    with _on(counts) as stream:
        st = lib.vsa_pack_lists(_ptr(counts), _ptr(ids_padded), n_rows, k_max, _ptr(offs), _ptr(ids),
                                stream)
    _lib.check("vsa_pack_lists", st)
    return offs, ids


def vsa_fine_forward(q, kp, vp, oc, gate_c, gate_f, grid, kv_ids, topk=0, kv_offsets=None,
                     out=None, save=False, order=None):
    """Fine stage + gated combine on raster q and K / V tiles; `order`
    (from vsa_fine_order) sets the order the query cubes run in.
    Returns (out, lse_f or None, o_fine or None)."""
    lib = _lib.load()
    B, N, nh, D, T, H, W, dt = _check_inputs(q, q, q, gate_c, gate_f, grid)
    nc = N // 64
    _need(kp, "kp", q.dtype, shape=(B, nh, nc, 64, D), device=q.device)
    _need(vp, "vp", q.dtype, shape=(B, nh, nc, 64, D), device=q.device)
    _need(oc, "oc", torch.float32, shape=(B, nh, nc, D), device=q.device)
    _need(kv_ids, "kv_ids", torch.int32, device=q.device)
    if kv_offsets is not None:
        _need(kv_offsets, "kv_offsets", torch.int32, numel=B * nh * nc + 1, device=q.device)
    elif kv_ids.numel() != B * nh * nc * topk:
        raise ValueError("kv_ids must hold B*heads*Nc*topk ids")
    if order is not None:
        _need(order, "order", torch.int32, numel=B * nh * nc, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", q.dtype, shape=q.shape, device=q.device)
    lse = of = None
    if save:
        lse = torch.empty((B, nh, N), dtype=torch.float32, device=q.device)
        of = torch.empty((B, nh, N, D), dtype=torch.float32, device=q.device)
    with _on(q) as stream:
        st = lib.vsa_fine_forward(_ptr(q), _ptr(kp), _ptr(vp), _ptr(oc), _ptr(gate_c), _ptr(gate_f),
                                  B, nh, D, *grid, _ptr(kv_offsets), _ptr(kv_ids), int(kv_ids.numel()), topk,
                                  _DT[q.dtype], _ptr(out), _ptr(lse), _ptr(of), _ptr(order), stream)
    _lib.check("vsa_fine_forward", st)
    return out, lse, of


def vsa_fine_order(kv_ids, B, heads, n_cubes, topk=0, kv_offsets=None):
    """Processing order for the fine stage (each (b, h)'s query cubes sorted
    by a Morton code of their lists' entries at indices n/4 and 3n/4).
    Returns int32 [B * heads * Nc]."""
    lib = _lib.load()
    _need(kv_ids, "kv_ids", torch.int32, device=kv_ids.device)
    if kv_offsets is not None:
        _need(kv_offsets, "kv_offsets", torch.int32, numel=B * heads * n_cubes + 1, device=kv_ids.device)
    elif kv_ids.numel() != B * heads * n_cubes * topk:
        raise ValueError("kv_ids must hold B*heads*Nc*topk ids")
    order = torch.empty(B * heads * n_cubes, dtype=torch.int32, device=kv_ids.device)
    with _on(kv_ids) as stream:
        st = lib.vsa_fine_order(_ptr(kv_offsets), _ptr(kv_ids), int(kv_ids.numel()), topk, B, heads,
                                n_cubes, _ptr(order), stream)
    _lib.check("vsa_fine_order", st)
    return order
