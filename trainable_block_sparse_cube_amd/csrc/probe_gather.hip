// Data-movement floor of the fine stage (see include/vsa_probe.h): the K
// and V tile reads of the fine kernel with no arithmetic, DEPTH tiles in
// flight per workgroup.  Measurement only.
#include <climits>

#include "vsa_probe.h"
#include "vsa_device.h"

namespace vsa {
namespace {

// CPT: 16-byte chunks per thread per tile (a tile is 8 * head_dim chunks).
template <int CPT, int DEPTH>
__global__ __launch_bounds__(256) void tile_gather_kernel(
    const u32x4* __restrict__ kp, const u32x4* __restrict__ vp, int nc,
    const int32_t* __restrict__ ids, int topk, int n_logical, u32x4* __restrict__ sink) {
  constexpr int TILE = 256 * CPT;
  // bh * nc + query cube, numbered XCD-contiguously as in the fine kernel
  const int per = (n_logical + 7) >> 3;
  const int64_t blk = (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (blk >= n_logical) return;
  const int64_t bh_tiles = (blk / nc) * nc;
  const int32_t* list = ids + blk * topk;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int t0 = 0; t0 < topk; t0 += DEPTH) {
    u32x4 r[DEPTH][2 * CPT];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (t0 + d < topk) {
        const int64_t base = (bh_tiles + list[t0 + d]) * TILE;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          r[d][j] = kp[base + j * 256 + threadIdx.x];
          r[d][CPT + j] = vp[base + j * 256 + threadIdx.x];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2 * CPT; ++j) r[d][j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
#pragma unroll
      for (int j = 0; j < 2 * CPT; ++j) acc ^= r[d][j];
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) sink[threadIdx.x] = acc;
}

template <int CPT>
hipError_t launch(const void* kp, const void* vp, int BH, int nc, const int32_t* ids, int topk,
                  int depth, void* sink, hipStream_t st) {
  const int n_logical = (int)((int64_t)BH * nc);
  const unsigned grid = ((unsigned)n_logical + 7u) / 8u * 8u;
  const u32x4* k = (const u32x4*)kp;
  const u32x4* v = (const u32x4*)vp;
  u32x4* s = (u32x4*)sink;
  switch (depth) {
    case 1: tile_gather_kernel<CPT, 1><<<grid, 256, 0, st>>>(k, v, nc, ids, topk, n_logical, s); break;
    case 2: tile_gather_kernel<CPT, 2><<<grid, 256, 0, st>>>(k, v, nc, ids, topk, n_logical, s); break;
    case 4: tile_gather_kernel<CPT, 4><<<grid, 256, 0, st>>>(k, v, nc, ids, topk, n_logical, s); break;
    default: tile_gather_kernel<CPT, 8><<<grid, 256, 0, st>>>(k, v, nc, ids, topk, n_logical, s); break;
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace vsa

extern "C" int vsa_probe_tile_gather(const void* kp, const void* vp, int BH, int n_cubes, int head_dim,
                                     const int32_t* ids, int topk, int depth, void* sink,
                                     hipStream_t stream) {
  if (!kp || !vp || !ids || !sink || BH < 1 || n_cubes < 1 || topk < 1 || topk > n_cubes) return 1;
  if (head_dim != 64 && head_dim != 128) return 1;
  if (depth != 1 && depth != 2 && depth != 4 && depth != 8) return 1;
  if ((int64_t)BH * n_cubes > INT_MAX) return 1;
  const hipError_t e = head_dim == 128
      ? vsa::launch<4>(kp, vp, BH, n_cubes, ids, topk, depth, sink, stream)
      : vsa::launch<2>(kp, vp, BH, n_cubes, ids, topk, depth, sink, stream);
  return e == hipSuccess ? 0 : 4;
}
