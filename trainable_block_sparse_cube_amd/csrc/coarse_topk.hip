// Coarse stage: dense cube-to-cube attention on the pooled tensors and the
// top-K key cubes of every query cube.
//
// [VSA-sum, Approach] ("Faster Video Diffusion with Trainable Sparse
// Attention", summary page): the pooled cubes attend densely to each other,
// giving a coarse output per cube, and the coarse scores pick the top-K
// critical key cubes of each query cube.  [VSA-sum, Limitations]: this
// selection is a separate step, not fused into the fine attention kernel.
//
// One workgroup (4 waves) owns 16 query cubes of one (batch, head):
//   1. logits S[r][j] = scale * <qc_r, kc_j> for every key cube j with fp32
//      MFMA (operands straight from L2); the 16 x Nc block of logits stays
//      in LDS;
//   2. per row (one wave per row): top-K by (logit desc, index asc) found
//      with a bitwise search for the K-th largest key plus a ballot-based
//      ordered compaction, which also emits the ids ascending; then the
//      softmax statistics, and S is overwritten by the probabilities;
//   3. Oc = P * vc with fp32 MFMA, vc operands read straight from L2.
// Everything is fp32: the ranking must match an fp64 reference exactly
// except at near-ties.
#include "vsa_device.h"
#include "vsa_launch.h"

namespace vsa {

namespace {

constexpr int kLdsBudget = 160 * 1024;

// Monotone map float -> uint32 (larger float, larger key); -0 maps as +0.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

typedef float f32x4v __attribute__((ext_vector_type(4)));

// Largest t such that at least k of the wave's 64 lane values are >= t
// (k in [1, 64]): greedy bitwise search, one ballot per bit.
__device__ __forceinline__ uint32_t kth_largest_of_lanes(uint32_t x, int k) {
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    if (__popcll(__ballot(x >= cand)) >= k) thr = cand;
  }
  return thr;
}

// Rank selection for one row held by one wave.  `keys` holds this lane's
// order keys of entries lane + 64 j (0 past the end; real order keys are
// never 0).  Writes the topk entries with the largest (key, -index) to
// out[0..topk), ascending by index.  `cand` is per-wave LDS scratch of
// 64 * MAXJ words.
//
// The K-th largest key is found by a bitwise search over a pruned candidate
// set: for K <= 64 the K-th largest of the 64 per-lane maxima is a lower
// bound on the row's K-th largest key (the lane maxima are row entries), so
// only entries at or above it take part.
template <int MAXJ>
__device__ __forceinline__ void select_row(const uint32_t (&keys)[MAXJ], int nc, int topk,
                                           int lane, uint32_t* __restrict__ cand,
                                           int32_t* __restrict__ out) {
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  uint32_t lo = 0;
  if (topk <= 64) {
    uint32_t lane_max = 0;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) lane_max = max(lane_max, keys[j]);
    lo = kth_largest_of_lanes(lane_max, topk);
  }
  // Compact the candidates (key >= lo) into LDS.
  int ncand = 0;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    if (64 * j < nc) {
      const bool in = keys[j] >= lo && keys[j] != 0u;
      const uint64_t m = __ballot(in);
      if (in) cand[ncand + __popcll(m & lt_mask)] = keys[j];
      ncand += __popcll(m);
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  // K-th largest key among the candidates.  The greedy search starts from
  // 0: for probes c <= lo every candidate counts (>= K of them, as in the
  // full row), for c > lo the candidates are all entries >= c, so every
  // decision matches a search over the whole row.
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = thr | (1u << bit);
    int cnt = 0;
    for (int i0 = 0; i0 < ncand; i0 += 64) {
      const int i = i0 + lane;
      cnt += __popcll(__ballot(i < ncand && cand[i] >= c));
    }
    if (cnt >= topk) thr = c;
  }
  int n_gt = 0;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j)
    if (64 * j < nc) n_gt += __popcll(__ballot(keys[j] > thr));
  const int need_eq = topk - n_gt;
  int base = 0, eq_seen = 0;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    if (64 * j < nc) {
      const int idx = 64 * j + lane;
      const bool valid = idx < nc;
      const bool gt = valid && keys[j] > thr;
      const bool eq = valid && keys[j] == thr;
      const uint64_t eq_mask = __ballot(eq);
      const bool take = gt || (eq && (eq_seen + __popcll(eq_mask & lt_mask)) < need_eq);
      const uint64_t take_mask = __ballot(take);
      const int pos = base + __popcll(take_mask & lt_mask);
      if (take && pos < topk) out[pos] = idx;
      base += __popcll(take_mask);
      eq_seen += __popcll(eq_mask);
    }
  }
}

// One workgroup: R = 16 query rows of one (batch, head), 4 waves.
// Matrix products use v_mfma_f32_16x16x4f32 (fp32 in, fp32 accumulate).
// Lane l of a 16x16x4 step supplies row/column l % 16 and k-slice l / 16.
template <int D, int MAXJ>
__global__ __launch_bounds__(256, 2) void coarse_topk_kernel(
    const float* __restrict__ qc, const float* __restrict__ kc,
    const float* __restrict__ vc, int nc, int topk, float scale,
    float* __restrict__ oc, float* __restrict__ lse, int32_t* __restrict__ sel) {
  constexpr int R = 16;
  constexpr int DQ = D / 4;          // head_dim slice per lane group
  constexpr int NB = D / 64;         // 16-column output blocks per wave
  extern __shared__ float lds[];
  const int s_pitch = (nc + 35) & ~3;  // room for a zero-padded last key block
  float* S = lds;                      // [R][s_pitch]
  uint32_t* cand_all = reinterpret_cast<uint32_t*>(S + R * s_pitch);  // [4][64 * MAXJ]

  const int bh = blockIdx.y;
  const int row0 = blockIdx.x * R;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, lg = lane >> 4;
  const float* qcb = qc + (int64_t)bh * nc * D;
  const float* kcb = kc + (int64_t)bh * nc * D;
  const float* vcb = vc + (int64_t)bh * nc * D;

  // ---- 1. logits.  Contraction over head_dim: lane group lg covers
  // d in [lg*DQ, lg*DQ + DQ), one element per k-step.  The next 16-key
  // block's operands are fetched while the current one is multiplied.
  f32x4v qa[DQ / 4];
  {
    const int row = min(row0 + li, nc - 1);  // rows past the end are never stored
    const f32x4v* src = reinterpret_cast<const f32x4v*>(qcb + (int64_t)row * D + lg * DQ);
#pragma unroll
    for (int i = 0; i < DQ / 4; ++i) qa[i] = src[i];
  }
  auto load_k = [&](int j0, f32x4v (&kb)[DQ / 4]) {
    const f32x4v* src = reinterpret_cast<const f32x4v*>(kcb + (int64_t)min(j0 + li, nc - 1) * D + lg * DQ);
#pragma unroll
    for (int i = 0; i < DQ / 4; ++i) kb[i] = src[i];
  };
  f32x4v kb[DQ / 4], kn[DQ / 4];
  if (16 * wave < nc) load_k(16 * wave, kn);
  for (int j0 = 16 * wave; j0 < nc; j0 += 64) {
#pragma unroll
    for (int i = 0; i < DQ / 4; ++i) kb[i] = kn[i];
    if (j0 + 64 < nc) load_k(j0 + 64, kn);
    f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < DQ / 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[i][e], kb[i][e], acc, 0, 0, 0);
    const int key = j0 + li;
    if (key < nc) {
#pragma unroll
      for (int r = 0; r < 4; ++r) S[(4 * lg + r) * s_pitch + key] = acc[r] * scale;
    }
  }
  __syncthreads();

  // ---- 2. per-row top-K and softmax, one wave per row
  for (int rr = wave; rr < R; rr += 4) {
    const int row = row0 + rr;
    float* Srow = S + rr * s_pitch;
    if (row >= nc) {  // keep padded rows finite for phase 3
      for (int j = lane; j < s_pitch; j += 64) Srow[j] = 0.f;
      continue;
    }
    if (topk > 0) {
      uint32_t keys[MAXJ];
#pragma unroll
      for (int j = 0; j < MAXJ; ++j) {
        const int idx = 64 * j + lane;
        keys[j] = idx < nc ? order_key(Srow[idx]) : 0u;
      }
      select_row<MAXJ>(keys, nc, topk, lane, cand_all + wave * 64 * MAXJ,
                       sel + ((int64_t)bh * nc + row) * topk);
    }
    float m = -INFINITY;
    for (int j = lane; j < nc; j += 64) m = fmaxf(m, Srow[j]);
    m = wave_max(m);
    // exp(x) as 2^(x log2 e): one v_exp_f32 per entry.
    const float m2 = m * kLog2e;
    float z = 0.f;
    for (int j = lane; j < nc; j += 64) z += __builtin_amdgcn_exp2f(fmaf(Srow[j], kLog2e, -m2));
    z = wave_sum(z);
    const float inv = 1.0f / z;
    for (int j = lane; j < s_pitch; j += 64)
      Srow[j] = j < nc ? __builtin_amdgcn_exp2f(fmaf(Srow[j], kLog2e, -m2)) * inv : 0.f;
    if (lane == 0) lse[(int64_t)bh * nc + row] = m + logf(z);
  }
  __syncthreads();

  // ---- 3. Oc = P * vc.  Wave w owns output columns [D/4 * w, +D/4) in
  // NB blocks of 16; contraction over keys, lane group lg taking key
  // j0 + 4t + lg at k-step t.  B operands come straight from L2 (vc of one
  // head is small), the next 32-key block prefetched during the current.
  f32x4v oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x4v{0.f, 0.f, 0.f, 0.f};
  const int col0 = (D / 4) * wave + li;
  auto load_v = [&](int j0, float (&vbuf)[8][NB]) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int key = min(j0 + 4 * t + lg, nc - 1);  // P is 0 past the end
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) vbuf[t][nb] = vcb[(int64_t)key * D + col0 + 16 * nb];
    }
  };
  float vb[8][NB], vn[8][NB];
  load_v(0, vn);
  for (int j0 = 0; j0 < nc; j0 += 32) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) vb[t][nb] = vn[t][nb];
    if (j0 + 32 < nc) load_v(j0 + 32, vn);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float pa = S[li * s_pitch + j0 + 4 * t + lg];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa, vb[t][nb], oacc[nb], 0, 0, 0);
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 4 * lg + r;
      if (row < nc) oc[((int64_t)bh * nc + row) * D + col0 + 16 * nb] = oacc[nb][r];
    }
}

size_t coarse_lds_bytes(int nc, int maxj) {
  const int s_pitch = (nc + 35) & ~3;
  return sizeof(float) * ((size_t)16 * s_pitch + (size_t)4 * 64 * maxj);
}

template <int D, int MAXJ>
hipError_t launch_coarse_dj(const CoarseArgs& a, hipStream_t st) {
  const size_t lds = coarse_lds_bytes(a.nc, MAXJ);
  auto kern = coarse_topk_kernel<D, MAXJ>;
  // Raise the dynamic LDS limit once per kernel instance (host-side call).
  static size_t lds_limit = 0;
  if (lds > lds_limit) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    lds_limit = lds;
  }
  dim3 grid((unsigned)((a.nc + 15) / 16), (unsigned)(a.B * a.heads));
  kern<<<grid, 256, lds, st>>>(a.qc, a.kc, a.vc, a.nc, a.topk, 1.0f / sqrtf((float)D),
                                a.oc, a.lse, a.sel);
  return hipGetLastError();
}

template <int D>
hipError_t launch_coarse_d(const CoarseArgs& a, hipStream_t st) {
  if (a.nc <= 16 * 64) return launch_coarse_dj<D, 16>(a, st);
  return launch_coarse_dj<D, 40>(a, st);
}

}  // namespace

int coarse_max_cubes(int D) {
  (void)D;
  // 16 rows of logits plus candidate scratch in LDS, and at most 40 key
  // chunks of 64 per row.
  const int by_lds = (int)((kLdsBudget / sizeof(float) - 4 * 64 * 40) / 16) - 35;
  return by_lds < 40 * 64 ? by_lds : 40 * 64;
}

hipError_t launch_coarse_topk(const CoarseArgs& a, hipStream_t st) {
  return a.D == 128 ? launch_coarse_d<128>(a, st) : launch_coarse_d<64>(a, st);
}

}  // namespace vsa
