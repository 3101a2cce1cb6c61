"""Seeded synthetic workloads for hierarchical video sparse attention.

This module only draws random inputs of the right shapes and distributions.
It holds none of the attention arithmetic and is shared, unchanged, by the
tests, the benchmark and the oracle-side checks.  The HIP library never
imports it.

Distribution (one recipe for every workload):
  * Q, K and V are each "a per-cube mean vector + per-token noise": for every
    (batch, head) and every 4x4x4 block of the latent grid one mean vector is
    drawn from N(0, 1); every token in the block adds its own N(0, 0.5^2)
    noise.  Q, K and V get independent means.
  * The two gates are sigmoid(N(0, 1)), one scalar per (batch, token, head).
  * The output cotangent dO (training workload) is N(0, 1).
  * Variable-length key-cube lists: for each (batch, head, query cube) a count
    L ~ UniformInt[lo, hi] and L distinct cube ids drawn without replacement,
    stored ascending.
  * bf16 workloads round the fp32 draws once, round-to-nearest-even; both the
    GPU path and the oracle consume those exact rounded values.

A second structure ("smooth", used only by the long61k_smooth extra): the
per-cube means vary smoothly over the cube grid instead of independently, a
stand-in for video, where neighbouring cubes look alike and so select
overlapping key cubes.  Per (batch, head, tensor) an N(0, 1) field over the
(T/4, H/4, W/4) cube grid and head_dim is box-filtered (3 taps, periodic)
SMOOTH_PASSES times along each grid axis and rescaled to unit standard
deviation over the whole draw; tokens add N(0, 0.5^2) noise as before.

Token order is raster: token (t, y, x) of a T x H x W grid sits at flat index
(t*H + y)*W + x, and tensors are [B, N, heads, head_dim] / [B, N, heads].
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    heads: int
    head_dim: int
    grid: tuple  # (T, H, W)
    topk: tuple  # one or more top-K values evaluated on this shape
    dtype: str  # "f32" or "bf16"
    seed: int
    varlen: Optional[tuple] = None  # (lo, hi) for per-query-cube list lengths
    backward: bool = False
    structure: str = "blocks"  # "blocks" (independent cube means) or "smooth"

    @property
    def N(self) -> int:
        T, H, W = self.grid
        return T * H * W

    @property
    def n_cubes(self) -> int:
        return self.N // 64


# The five workloads.  Seeds are 1000 + index.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 2, 64, (8, 8, 8), (2,), "f32", 1000),
    "pretrain16k": Workload("pretrain16k", 1, 12, 128, (16, 32, 32), (32,), "bf16", 1001),
    "long61k": Workload("long61k", 1, 12, 128, (20, 48, 64), (16, 32), "bf16", 1002),
    "large70k": Workload("large70k", 1, 40, 128, (20, 44, 80), (32,), "bf16", 1003,
                         varlen=(8, 64)),
    "train16k": Workload("train16k", 2, 12, 128, (16, 32, 32), (32,), "bf16", 1004,
                         backward=True),
    # not one of the five: the headline shape with spatially smooth cube means
    "long61k_smooth": Workload("long61k_smooth", 1, 12, 128, (20, 48, 64), (32,), "bf16", 1005,
                               structure="smooth"),
}

SMOOTH_PASSES = 4


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of fp32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _blockwise_mean_plus_noise(rng, B, T, H, W, heads, D, noise_std):
    """[B, T*H*W, heads, D]: one N(0,1) vector per 4x4x4 block + token noise."""
    mean = rng.standard_normal((B, T // 4, H // 4, W // 4, heads, D), dtype=np.float32)
    full = np.broadcast_to(
        mean[:, :, None, :, None, :, None, :, :],
        (B, T // 4, 4, H // 4, 4, W // 4, 4, heads, D),
    ).reshape(B, T * H * W, heads, D)
    noise = rng.standard_normal((B, T * H * W, heads, D), dtype=np.float32)
    return (full + np.float32(noise_std) * noise).astype(np.float32)


def _smooth_mean_plus_noise(rng, B, T, H, W, heads, D, noise_std):
    """[B, T*H*W, heads, D]: a smooth field of cube means + token noise."""
    f = rng.standard_normal((B, T // 4, H // 4, W // 4, heads, D), dtype=np.float32)
    for axis in (1, 2, 3):
        for _ in range(SMOOTH_PASSES):
            f = (f + np.roll(f, 1, axis=axis) + np.roll(f, -1, axis=axis)) / np.float32(3.0)
    f = (f / f.std()).astype(np.float32)
    full = np.broadcast_to(
        f[:, :, None, :, None, :, None, :, :],
        (B, T // 4, 4, H // 4, 4, W // 4, 4, heads, D),
    ).reshape(B, T * H * W, heads, D)
    noise = rng.standard_normal((B, T * H * W, heads, D), dtype=np.float32)
    return (full + np.float32(noise_std) * noise).astype(np.float32)


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def make_inputs(B, heads, D, grid, dtype="bf16", seed=0, with_dout=False,
                varlen=None, structure="blocks"):
    """Draw one seeded input set.

    Returns a dict of fp32 numpy arrays (bf16-exact when dtype == "bf16"):
      q, k, v: [B, N, heads, D]; gc, gf: [B, N, heads]; optionally
      dout: [B, N, heads, D]; and for varlen=(lo, hi): kv_offsets int32
      [B*heads*Nc + 1] and kv_ids int32, lists ordered by (b, h, query cube).
    """
    T, H, W = grid
    if T % 4 or H % 4 or W % 4:
        raise ValueError("grid dimensions must be multiples of 4")
    rng = np.random.default_rng(seed)
    out = {}
    draw = {"blocks": _blockwise_mean_plus_noise, "smooth": _smooth_mean_plus_noise}[structure]
    for name in ("q", "k", "v"):
        out[name] = draw(rng, B, T, H, W, heads, D, 0.5)
    N = T * H * W
    out["gc"] = _sigmoid(rng.standard_normal((B, N, heads), dtype=np.float32))
    out["gf"] = _sigmoid(rng.standard_normal((B, N, heads), dtype=np.float32))
    if with_dout:
        out["dout"] = rng.standard_normal((B, N, heads, D), dtype=np.float32)
    if varlen is not None:
        lo, hi = varlen
        nc = N // 64
        counts = rng.integers(lo, hi + 1, size=B * heads * nc)
        counts = np.minimum(counts, nc)
        ids = []
        for cnt in counts:
            ids.append(np.sort(rng.choice(nc, size=int(cnt), replace=False)))
        offs = np.zeros(B * heads * nc + 1, dtype=np.int64)
        offs[1:] = np.cumsum(counts)
        out["kv_offsets"] = offs.astype(np.int32)
        out["kv_ids"] = (np.concatenate(ids) if ids else np.zeros(0)).astype(np.int32)
    if dtype == "bf16":
        for name in ("q", "k", "v", "gc", "gf", "dout"):
            if name in out:
                out[name] = round_to_bf16(out[name])
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype}")
    return out


def workload_inputs(w: Workload, seed=None, with_varlen=True):
    return make_inputs(w.B, w.heads, w.head_dim, w.grid, w.dtype,
                       w.seed if seed is None else seed,
                       with_dout=w.backward,
                       varlen=w.varlen if with_varlen else None,
                       structure=w.structure)


def fine_flops(B, heads, N, topk, D):
    """Effective (sparse) FLOPs of the fine-stage forward: QK^T and PV, each
    2*D per (query token, selected key token); topk cubes of 64 tokens."""
    return 4.0 * B * heads * N * topk * 64 * D


def fine_flops_lists(total_list_entries, D):
    """Same count for variable-length lists: every list entry pairs the 64
    query tokens of a cube with the 64 key tokens of one selected cube."""
    return 4.0 * 64 * 64 * D * float(total_list_entries)


def coarse_flops(B, heads, n_cubes, D):
    """Dense cube-to-cube attention on pooled tensors: QK^T and PV."""
    return 4.0 * B * heads * n_cubes * n_cubes * D
