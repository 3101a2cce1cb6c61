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
//   3. Oc = P * vc with fp32 MFMA, vc streamed through LDS.
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

__device__ __forceinline__ int wave_sum_i(int x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

typedef float f32x4v __attribute__((ext_vector_type(4)));

// One workgroup: R = 16 query rows of one (batch, head), 4 waves.
// Matrix products use v_mfma_f32_16x16x4f32 (fp32 in, fp32 accumulate).
// Lane l of a 16x16x4 step supplies row/column l % 16 and k-slice l / 16.
template <int D>
__global__ __launch_bounds__(256, 2) void coarse_topk_kernel(
    const float* __restrict__ qc, const float* __restrict__ kc,
    const float* __restrict__ vc, int nc, int topk, float scale,
    float* __restrict__ oc, float* __restrict__ lse, int32_t* __restrict__ sel) {
  constexpr int R = 16;
  constexpr int DQ = D / 4;          // head_dim slice per lane group
  constexpr int VCH = 16;            // value rows per LDS chunk
  constexpr int VPITCH = D + 4;
  extern __shared__ float lds[];
  const int s_pitch = (nc + 19) & ~3;  // room for a zero-padded last value chunk
  float* S = lds;                      // [R][s_pitch]
  float* vch = S + R * s_pitch;        // [VCH][VPITCH]

  const int bh = blockIdx.y;
  const int row0 = blockIdx.x * R;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, lg = lane >> 4;
  const float* qcb = qc + (int64_t)bh * nc * D;
  const float* kcb = kc + (int64_t)bh * nc * D;
  const float* vcb = vc + (int64_t)bh * nc * D;

  // ---- 1. logits.  Contraction over head_dim: lane group lg covers
  // d in [lg*DQ, lg*DQ + DQ), one element per k-step.
  f32x4v qa[DQ / 4];
  {
    const int row = min(row0 + li, nc - 1);  // rows past the end are never stored
    const f32x4v* src = reinterpret_cast<const f32x4v*>(qcb + (int64_t)row * D + lg * DQ);
#pragma unroll
    for (int i = 0; i < DQ / 4; ++i) qa[i] = src[i];
  }
  for (int j0 = 16 * wave; j0 < nc; j0 += 64) {
    const int key = j0 + li;
    const f32x4v* src = reinterpret_cast<const f32x4v*>(kcb + (int64_t)min(key, nc - 1) * D + lg * DQ);
    f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < DQ / 4; ++i) {
      const f32x4v kb = src[i];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[i][e], kb[e], acc, 0, 0, 0);
    }
    if (key < nc) {
#pragma unroll
      for (int r = 0; r < 4; ++r) S[(4 * lg + r) * s_pitch + key] = acc[r] * scale;
    }
  }
  __syncthreads();

  // ---- 2. per-row top-K and softmax, one wave per row
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  for (int rr = wave; rr < R; rr += 4) {
    const int row = row0 + rr;
    float* Srow = S + rr * s_pitch;
    if (row >= nc) {  // keep padded rows finite for phase 3
      for (int j = lane; j < s_pitch; j += 64) Srow[j] = 0.f;
      continue;
    }
    if (topk > 0) {
      uint32_t thr = 0;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = thr | (1u << bit);
        int cnt = 0;
        for (int j = lane; j < nc; j += 64) cnt += order_key(Srow[j]) >= cand;
        if (wave_sum_i(cnt) >= topk) thr = cand;
      }
      int n_gt = 0;
      for (int j = lane; j < nc; j += 64) n_gt += order_key(Srow[j]) > thr;
      const int need_eq = topk - wave_sum_i(n_gt);
      int32_t* out = sel + ((int64_t)bh * nc + row) * topk;
      int base = 0, eq_seen = 0;
      for (int jb = 0; jb < nc; jb += 64) {
        const int j = jb + lane;
        const uint32_t key = j < nc ? order_key(Srow[j]) : 0u;
        const bool gt = j < nc && key > thr;
        const bool eq = j < nc && key == thr;
        const uint64_t eq_mask = __ballot(eq);
        const bool take = gt || (eq && (eq_seen + __popcll(eq_mask & lt_mask)) < need_eq);
        const uint64_t take_mask = __ballot(take);
        const int pos = base + __popcll(take_mask & lt_mask);
        if (take && pos < topk) out[pos] = j;
        base += __popcll(take_mask);
        eq_seen += __popcll(eq_mask);
      }
    }
    float m = -INFINITY;
    for (int j = lane; j < nc; j += 64) m = fmaxf(m, Srow[j]);
    m = wave_max(m);
    float z = 0.f;
    for (int j = lane; j < nc; j += 64) z += expf(Srow[j] - m);
    z = wave_sum(z);
    const float inv = 1.0f / z;
    for (int j = lane; j < s_pitch; j += 64) Srow[j] = j < nc ? expf(Srow[j] - m) * inv : 0.f;
    if (lane == 0) lse[(int64_t)bh * nc + row] = m + logf(z);
  }

  // ---- 3. Oc = P * vc.  Wave w owns output columns [32w, 32w + 32)
  // (two 16-column blocks; D = 64 uses one); contraction over keys with
  // lane group lg taking key j0 + 4t + lg at k-step t.
  constexpr int NB = D / 64;  // 16-column blocks per wave
  f32x4v oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x4v{0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < nc; j0 += VCH) {
    __syncthreads();
    for (int i = tid; i < VCH * (D / 4); i += 256) {
      const int j = i / (D / 4), d4 = i % (D / 4);
      f32x4v val = {0.f, 0.f, 0.f, 0.f};
      if (j0 + j < nc) val = reinterpret_cast<const f32x4v*>(vcb + (int64_t)(j0 + j) * D)[d4];
      *reinterpret_cast<f32x4v*>(&vch[j * VPITCH + 4 * d4]) = val;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < VCH / 4; ++t) {
      const int j = 4 * t + lg;
      const float pa = S[li * s_pitch + j0 + j];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(
            pa, vch[j * VPITCH + (D / 4) * wave + 16 * nb + li], oacc[nb], 0, 0, 0);
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 4 * lg + r;
      if (row < nc) oc[((int64_t)bh * nc + row) * D + (D / 4) * wave + 16 * nb + li] = oacc[nb][r];
    }
}

size_t coarse_lds_bytes(int D, int nc) {
  const int s_pitch = (nc + 19) & ~3;
  return sizeof(float) * ((size_t)16 * s_pitch + (size_t)16 * (D + 4));
}

template <int D>
hipError_t launch_coarse_d(const CoarseArgs& a, hipStream_t st) {
  const size_t lds = coarse_lds_bytes(D, a.nc);
  auto kern = coarse_topk_kernel<D>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((a.nc + 15) / 16), (unsigned)(a.B * a.heads));
  kern<<<grid, 256, lds, st>>>(a.qc, a.kc, a.vc, a.nc, a.topk, 1.0f / sqrtf((float)D),
                                a.oc, a.lse, a.sel);
  return hipGetLastError();
}

}  // namespace

int coarse_max_cubes(int D) {
  // 16 rows of logits (padded) and one 16-row value chunk must fit in LDS.
  const size_t rows = (kLdsBudget / sizeof(float) - 16 * (size_t)(D + 4)) / 16;
  return (int)rows - 19;
}

hipError_t launch_coarse_topk(const CoarseArgs& a, hipStream_t st) {
  return a.D == 128 ? launch_coarse_d<128>(a, st) : launch_coarse_d<64>(a, st);
}

}  // namespace vsa
