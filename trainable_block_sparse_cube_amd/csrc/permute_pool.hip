// Cube permute + mean pooling (one pass over Q, K, V).
//
// [VSA-sum, Approach] ("Faster Video Diffusion with Trainable Sparse
// Attention", summary page): tokens are grouped into 4x4x4 cubes, each cube
// is one tile of the fine stage, and Q/K/V are mean-pooled per cube for the
// coarse stage.  One workgroup handles one (batch, cube, head) of one tensor:
// it gathers the cube's 64 token rows (each row D contiguous elements in the
// raster layout), writes them as one contiguous cube-major tile, and reduces
// the 64 rows to their fp32 mean with wavefront shuffles plus a 4-way LDS
// combine.  The forward writes the K and V tiles (the fine stage reads Q in
// place); the backward writes Q tiles only (it reads the K and V tiles and
// the cube means the forward left in its saved state, which the forward
// writes as a second, plain-layout copy of the K and V means when its own
// copy is packed).  The forward's bf16 path
// stores the pooled K and V in the coarse kernel's operand order (packed
// layouts, zero-padded keys).  A second instance takes
// the per-channel maximum instead of the mean and writes no tiles: the
// pooling ablation ([VSA-sum, Surprising findings]: mean pooling did better
// than max pooling).  Both reductions are exact in fp32 (the mean's sum of
// 64 values rounds per addition, like any fp32 sum).
#include "vsa_device.h"
#include "vsa_launch.h"

namespace vsa {

template <typename T, int D, bool MAXP, bool NT>
__global__ __launch_bounds__(256) void permute_pool_kernel(PermutePoolPtrs p, int nh, int Tg, int Hg, int Wg,
                                                           bool packed_kv) {
  constexpr int EPC = 16 / sizeof(T);     // elements per 16-byte chunk
  constexpr int CPR = D / EPC;            // chunks per token row
  constexpr int ROWS_PER_PASS = 256 / CPR;
  constexpr int PASSES = kCubeTokens / ROWS_PER_PASS;
  static_assert(256 % CPR == 0 && kCubeTokens % ROWS_PER_PASS == 0, "tiling");

  __shared__ float red[4][D];

  const int which = blockIdx.y;  // 0: q, 1: k, 2: v
  const T* __restrict__ src = (const T*)p.src[which];
  T* __restrict__ nat = (T*)p.nat[which];
  float* __restrict__ pooled = p.pooled[which];

  const int nc = (Tg / 4) * (Hg / 4) * (Wg / 4);
  const int N = Tg * Hg * Wg;
  const int h = blockIdx.x % nh;
  const int bc = blockIdx.x / nh;
  const int c = bc % nc;
  const int b = bc / nc;
  const int W4 = Wg / 4, H4 = Hg / 4;
  const int ct = c / (H4 * W4), cy = (c / W4) % H4, cx = c % W4;
  const int64_t tile = ((int64_t)(b * nh + h) * nc + c) * kCubeTokens * D;

  const int tid = threadIdx.x;
  const int ch = tid % CPR;  // this thread's chunk column, fixed over passes
  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = MAXP ? -INFINITY : 0.f;

#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int s = tid / CPR + ps * ROWS_PER_PASS;  // slot in cube
    const int tok = ((4 * ct + (s >> 4)) * Hg + 4 * cy + ((s >> 2) & 3)) * Wg + 4 * cx + (s & 3);
    const T* rowp = src + ((int64_t)b * N + tok) * nh * D + (int64_t)h * D;
    // Non-temporal load: each input row streams through here once, and
    // keeping it out of the caches leaves room for the tiles just written
    // (the whole forward measured about 1 % faster than with plain loads).
    const u32x4 raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowp + ch * EPC));
    T vals[EPC];
    __builtin_memcpy(vals, &raw, 16);
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = MAXP ? fmaxf(acc[e], to_f32(vals[e])) : acc[e] + to_f32(vals[e]);
    // Tiles that together overflow the last-level cache (MALL) are written
    // with non-temporal stores, the others with plain ones (see the launch).
    if (nat) {
      u32x4* dst = reinterpret_cast<u32x4*>(nat + tile + (int64_t)s * D + ch * EPC);
      if constexpr (NT) __builtin_nontemporal_store(raw, dst);
      else *dst = raw;
    }
  }

  if (pooled) {
    // Sum over the lanes of this wave that hold the same chunk column.
#pragma unroll
    for (int o = CPR; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const float other = __shfl_xor(acc[e], o);
        acc[e] = MAXP ? fmaxf(acc[e], other) : acc[e] + other;
      }
    const int wave = tid >> 6, lane = tid & 63;
    if (lane < CPR) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) red[wave][lane * EPC + e] = acc[e];
    }
  }
  __syncthreads();
  if (pooled) {
    const bool pk = packed_kv && which > 0;
    const int ncp = packed_keys(nc);
    float* base = pooled + (int64_t)(b * nh + h) * (pk ? ncp : nc) * D;
    float* plain = p.plain[which] ? p.plain[which] + ((int64_t)(b * nh + h) * nc + c) * D : nullptr;
    for (int d = tid; d < D; d += 256) {
      const float r = MAXP ? fmaxf(fmaxf(red[0][d], red[1][d]), fmaxf(red[2][d], red[3][d]))
                           : ((red[0][d] + red[1][d]) + (red[2][d] + red[3][d])) * (1.0f / kCubeTokens);
      if (!pk) base[(int64_t)c * D + d] = r;
      else if (which == 1) base[packed_k_index(c, d, D)] = r;
      else base[packed_v_index(c, d, D)] = r;
      if (plain) plain[d] = r;
    }
    if (pk && c == nc - 1) {  // zero the padding keys of this (b, h)
      for (int i = tid; i < (ncp - nc) * D; i += 256) {
        const int j = nc + i / D, d = i % D;
        base[which == 1 ? packed_k_index(j, d, D) : packed_v_index(j, d, D)] = 0.f;
      }
    }
  }
}

// Tile bytes a launch writes above which the stores bypass the caches: the
// 256 MB MALL of MI355X.  Measured on the permute stage alone: 61440 tokens,
// 12 heads, K and V tiles (378 MB): 0.174 ms non-temporal against 0.185
// plain; 16384 tokens (100 and 200 MB): 0.051 against 0.043 and 0.092
// against 0.079 ms; 300 MB (Q, K and V at B = 2): a tie.
constexpr double kNonTemporalTileBytes = 256.0 * 1024 * 1024;

template <typename T, int D>
static hipError_t launch_pp(const PermutePoolArgs& a, hipStream_t st) {
  const int nc = (a.T / 4) * (a.H / 4) * (a.W / 4);
  dim3 grid((unsigned)(a.B * nc * a.heads), (unsigned)a.n_tensors);
  if (a.max_pool) {
    PermutePoolPtrs p = a.p;
    p.nat[0] = p.nat[1] = p.nat[2] = nullptr;  // pooled values only
    p.plain[0] = p.plain[1] = p.plain[2] = nullptr;
    permute_pool_kernel<T, D, true, false><<<grid, 256, 0, st>>>(p, a.heads, a.T, a.H, a.W, false);
    return hipGetLastError();
  }
  int n_tiles = 0;
  for (int i = 0; i < a.n_tensors; ++i) n_tiles += a.p.nat[i] != nullptr;
  const double tile_bytes = (double)n_tiles * a.B * a.heads * nc * kCubeTokens * D * sizeof(T);
  if (tile_bytes > kNonTemporalTileBytes)
    permute_pool_kernel<T, D, false, true><<<grid, 256, 0, st>>>(a.p, a.heads, a.T, a.H, a.W, a.packed_kv);
  else
    permute_pool_kernel<T, D, false, false><<<grid, 256, 0, st>>>(a.p, a.heads, a.T, a.H, a.W, a.packed_kv);
  return hipGetLastError();
}

hipError_t launch_permute_pool(const PermutePoolArgs& a, hipStream_t st) {
  if (a.bf16) return a.D == 128 ? launch_pp<bf16, 128>(a, st) : launch_pp<bf16, 64>(a, st);
  return a.D == 128 ? launch_pp<float, 128>(a, st) : launch_pp<float, 64>(a, st);
}

}  // namespace vsa
