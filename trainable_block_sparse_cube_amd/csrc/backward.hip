// Backward of the whole operator: gradients of sum(dO * O) with respect to
// q, k, v and both gates, the selection held fixed.
//
// [VSA-abs] ("VSA: Faster Video Diffusion with Trainable Sparse Attention",
// Abstract): the operator is one differentiable kernel trained end to end.
// [VSA-sum, Approach]: O = g_c * Oc[cube] + g_f * O_fine, Oc from dense
// attention on cube means, O_fine from attention over the selected cubes.
// The top-K choice is piecewise constant, so no gradient flows through it;
// the coarse stage carries gradient to the cube means, and the mean spreads
// it evenly (1/64) over each cube's tokens.
//
// Kernels, in launch order (all deterministic, no atomics on floats):
//   bwd_prep        per (cube, head): dg_c = dO.Oc, dg_f = dO.O_fine (fp32),
//                   Delta = dOf.O_fine, dOf = g_f dO (bf16, natural and
//                   transposed tiles), dOc = sum over the cube of g_c dO and
//                   Delta_c = dOc.Oc
//   gemm_f32 / coarse_softmax_grad
//                   coarse backward on the means: S, dP by fp32 MFMA GEMMs,
//                   P = exp(S - lse_c), dS = P (dP - Delta_c), then
//                   dQc = s dS Kc, dKc = s dS^T Qc, dVc = P^T dOc
//   transpose_lists for every key cube, the ascending list of query cubes
//                   that selected it (counting sort + per-list sort)
//   fine_bwd_dkdv   key-stationary: one workgroup per key cube accumulates
//                   dK and dV over the query cubes that selected it
//   fine_bwd_dq     query-stationary: one workgroup per query cube
//                   accumulates dQ over its selected key cubes
// The last two write raster-order gradients with the coarse share added.
#include "vsa_device.h"
#include "vsa_launch.h"

namespace vsa {

namespace {

__device__ __forceinline__ int raster_tok(int c, int s, int Hg, int Wg) {
  const int W4 = Wg >> 2, H4 = Hg >> 2;
  const int ct = c / (H4 * W4), cy = (c / W4) % H4, cx = c % W4;
  return ((4 * ct + (s >> 4)) * Hg + 4 * cy + ((s >> 2) & 3)) * Wg + 4 * cx + (s & 3);
}

// ---------------------------------------------------------------- prep
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(
    const bf16* __restrict__ dout, const bf16* __restrict__ gc, const bf16* __restrict__ gf,
    const float* __restrict__ of, const float* __restrict__ oc, int nh, int Tg, int Hg, int Wg,
    float* __restrict__ dgc, float* __restrict__ dgf, float* __restrict__ delta,
    bf16* __restrict__ dofp, bf16* __restrict__ doft, float* __restrict__ doc,
    float* __restrict__ deltac) {
  constexpr int EPC = 8;
  constexpr int CPR = D / EPC;
  constexpr int RPP = 256 / CPR;
  constexpr int PASSES = kCubeTokens / RPP;
  constexpr int PITCH = kCubeTokens + EPC;
  __shared__ __align__(16) bf16 t_lds[D * PITCH];
  __shared__ float red[4][D];
  __shared__ float dsum[D];

  const int nc = (Tg / 4) * (Hg / 4) * (Wg / 4);
  const int N = Tg * Hg * Wg;
  const int h = blockIdx.x % nh;
  const int bc = blockIdx.x / nh;
  const int c = bc % nc;
  const int b = bc / nc;
  const int bh = b * nh + h;
  const int64_t tile = ((int64_t)bh * nc + c) * kCubeTokens * D;
  const int tid = threadIdx.x;
  const int ch = tid % CPR;

  float ocv[EPC];
  {
    const f32x4* p = reinterpret_cast<const f32x4*>(oc + ((int64_t)bh * nc + c) * D + ch * EPC);
    const f32x4 a = p[0], bb = p[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) { ocv[e] = a[e]; ocv[4 + e] = bb[e]; }
  }
  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.f;

#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int s = tid / CPR + ps * RPP;
    const int tok = raster_tok(c, s, Hg, Wg);
    const int64_t gidx = ((int64_t)b * N + tok) * nh + h;
    const u32x4 raw = *reinterpret_cast<const u32x4*>(dout + gidx * D + ch * EPC);
    bf16 gv[EPC];
    __builtin_memcpy(gv, &raw, 16);
    const float gcs = (float)gc[gidx], gfs = (float)gf[gidx];
    const f32x4* op = reinterpret_cast<const f32x4*>(of + ((int64_t)bh * N + (int64_t)c * 64 + s) * D + ch * EPC);
    const f32x4 o0 = op[0], o1 = op[1];
    // pc, pf: dO.Oc and dO.O_fine (the gate gradients, fp32).  pd is
    // Delta = dOf.O_fine taken with dOf rounded to bf16 exactly as the fine
    // kernels use it, so that sum_j P_ij dP_ij = Delta_i holds to fp32
    // accuracy and dS sums to zero over each row.
    float pc = 0.f, pf = 0.f, pd = 0.f;
    bf16 dv[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const float g = (float)gv[e];
      const float ofe = e < 4 ? o0[e] : o1[e - 4];
      pc = fmaf(g, ocv[e], pc);
      pf = fmaf(g, ofe, pf);
      acc[e] = fmaf(gcs, g, acc[e]);
      dv[e] = (bf16)(gfs * g);
      pd = fmaf((float)dv[e], ofe, pd);
    }
#pragma unroll
    for (int o = 1; o < CPR; o <<= 1) {
      pc += __shfl_xor(pc, o);
      pf += __shfl_xor(pf, o);
      pd += __shfl_xor(pd, o);
    }
    if (ch == 0) {
      dgc[gidx] = pc;
      dgf[gidx] = pf;
      delta[(int64_t)bh * N + (int64_t)c * 64 + s] = pd;
    }
    u32x4 packed;
    __builtin_memcpy(&packed, dv, 16);
    *reinterpret_cast<u32x4*>(dofp + tile + (int64_t)s * D + ch * EPC) = packed;
    const int pos = vt_key_of_pos(s);
#pragma unroll
    for (int e = 0; e < EPC; ++e) t_lds[(ch * EPC + e) * PITCH + pos] = dv[e];
  }
#pragma unroll
  for (int o = CPR; o < 64; o <<= 1)
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] += __shfl_xor(acc[e], o);
  const int wave = tid >> 6, lane = tid & 63;
  if (lane < CPR) {
#pragma unroll
    for (int e = 0; e < EPC; ++e) red[wave][lane * EPC + e] = acc[e];
  }
  __syncthreads();
  if (tid < D) {
    const float v = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
    doc[((int64_t)bh * nc + c) * D + tid] = v;
    dsum[tid] = v * oc[((int64_t)bh * nc + c) * D + tid];
  }
  constexpr int VCPR = kCubeTokens / EPC;
  for (int i = tid; i < D * VCPR; i += 256) {
    const int d = i / VCPR, cc = i % VCPR;
    *reinterpret_cast<u32x4*>(doft + tile + (int64_t)d * kCubeTokens + cc * EPC) =
        *reinterpret_cast<const u32x4*>(&t_lds[d * PITCH + cc * EPC]);
  }
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int d = 0; d < D; ++d) t += dsum[d];
    deltac[(int64_t)bh * nc + c] = t;
  }
}

// ---------------------------------------------------------------- coarse
typedef float f32x4v __attribute__((ext_vector_type(4)));

// C[z] = alpha * op(A[z]) * op(B[z]) for z < batch, fp32, row-major.
// op(A) is M x K (TA: A stored K x M); op(B) is K x N (TB: B stored N x K).
// 64 x 64 output tile per workgroup, 16-deep K chunks staged in LDS,
// v_mfma_f32_16x16x4f32; each wave owns a 32 x 32 quarter.
template <bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float* __restrict__ A, int lda, int64_t sA, const float* __restrict__ B, int ldb, int64_t sB,
    float* __restrict__ C, int ldc, int64_t sC, int M, int N, int K, float alpha) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int z = blockIdx.z;
  A += z * sA; B += z * sB; C += z * sC;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  f32x4v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += 16) {
    __syncthreads();
    for (int i = tid; i < 16 * 64; i += 256) {
      int kk, mm;
      if (TA) { kk = i / 64; mm = i % 64; } else { mm = i / 16; kk = i % 16; }
      const int gm = m0 + mm, gk = k0 + kk;
      As[kk][mm] = (gm < M && gk < K) ? (TA ? A[(int64_t)gk * lda + gm] : A[(int64_t)gm * lda + gk]) : 0.f;
      int nn;
      if (TB) { nn = i / 16; kk = i % 16; } else { kk = i / 64; nn = i % 64; }
      const int gn = n0 + nn; const int gk2 = k0 + kk;
      Bs[kk][nn] = (gn < N && gk2 < K) ? (TB ? B[(int64_t)gn * ldb + gk2] : B[(int64_t)gk2 * ldb + gn]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kk = 4 * t + lg;
      float a[2], bb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = As[kk][32 * wm + 16 * i + li];
#pragma unroll
      for (int j = 0; j < 2; ++j) bb[j] = Bs[kk][32 * wn + 16 * j + li];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], bb[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gm = m0 + 32 * wm + 16 * i + 4 * lg + r;
        const int gn = n0 + 32 * wn + 16 * j + li;
        if (gm < M && gn < N) C[(int64_t)gm * ldc + gn] = alpha * acc[i][j][r];
      }
}

// Row-wise: P = exp(S - lse), dS = P * (dP - Delta_c); S and dP [rows][nc]
// (already scaled logits), overwritten by P and dS.
__global__ __launch_bounds__(256) void coarse_softmax_grad_kernel(
    float* __restrict__ S, float* __restrict__ dP, const float* __restrict__ lse,
    const float* __restrict__ deltac, int nc, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const float l = lse[row], dl = deltac[row];
  float* s = S + row * nc;
  float* dp = dP + row * nc;
  for (int j = lane; j < nc; j += 64) {
    const float p = expf(s[j] - l);
    s[j] = p;
    dp[j] = p * (dp[j] - dl);
  }
}

// ---------------------------------------------------------------- lists
// For every (b, h) and key cube j: tr_ids[tr_offs[r] .. tr_offs[r+1]) are
// the query cubes whose list contains j, ascending (r = (b*nh + h)*nc + j).
// Lists: CSR (offs) or fixed length topk (offs == null).  The output of
// (b, h) occupies the same index range as its input lists.
__global__ __launch_bounds__(256) void transpose_lists_kernel(
    const int32_t* __restrict__ offs, const int32_t* __restrict__ ids, int topk, int nc,
    int32_t* __restrict__ tr_offs, int32_t* __restrict__ tr_ids) {
  extern __shared__ int32_t cnt[];  // [nc] counts, then [nc + 1] starts
  int32_t* start = cnt + nc;
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)bh * nc;
  const int base = offs ? offs[r0] : (int)(r0 * topk);
  const int total = (offs ? offs[r0 + nc] : (int)((r0 + nc) * topk)) - base;
  for (int j = tid; j < nc; j += 256) cnt[j] = 0;
  __syncthreads();
  for (int e = tid; e < total; e += 256) {
    const int j = ids[base + e];
    if (j >= 0 && j < nc) atomicAdd(&cnt[j], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int j = 0; j < nc; ++j) { start[j] = run; run += cnt[j]; }
    start[nc] = run;
  }
  __syncthreads();
  for (int j = tid; j <= nc; j += 256) tr_offs[r0 + j] = base + start[j];
  for (int j = tid; j < nc; j += 256) cnt[j] = start[j];  // fill cursors
  __syncthreads();
  for (int c = tid; c < nc; c += 256) {
    const int e0 = offs ? offs[r0 + c] : (int)((r0 + c) * topk);
    const int e1 = offs ? offs[r0 + c + 1] : e0 + topk;
    for (int e = e0; e < e1; ++e) {
      const int j = ids[e];
      if (j >= 0 && j < nc) tr_ids[base + atomicAdd(&cnt[j], 1)] = c;
    }
  }
  __syncthreads();
  for (int j = tid; j < nc; j += 256) {  // insertion sort of each list
    int32_t* l = tr_ids + base + start[j];
    const int n = start[j + 1] - start[j];
    for (int i = 1; i < n; ++i) {
      const int32_t x = l[i];
      int k = i - 1;
      while (k >= 0 && l[k] > x) { l[k + 1] = l[k]; --k; }
      l[k + 1] = x;
    }
  }
}

// ---------------------------------------------------------------- fine
template <int D>
__device__ __forceinline__ int swz_row(int row) {
  if constexpr (D == 128) return row & 15;
  else return (row ^ (row >> 3)) & 7;
}
__device__ __forceinline__ int swz_t(int row) { return (row ^ (row >> 3)) & 7; }

// Stage one natural tile [64][D] (swizzled chunks) and one transposed tile
// [D][64] (MFMA token order, swizzled chunks) into LDS with plain loads.
template <int D, int NT>
__device__ __forceinline__ void stage_nat(const bf16* __restrict__ src, u32x4* dst, int tid) {
  constexpr int KCH = D / 8;
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  for (int i = tid; i < 64 * KCH; i += NT) {
    const int row = i / KCH, chk = i % KCH;
    dst[row * KCH + (chk ^ swz_row<D>(row))] = s[i];
  }
}
template <int D, int NT>
__device__ __forceinline__ void stage_tr(const bf16* __restrict__ src, u32x4* dst, int tid) {
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  for (int i = tid; i < D * 8; i += NT) {
    const int row = i >> 3, chk = i & 7;
    dst[row * 8 + (chk ^ swz_t(row))] = s[i];
  }
}

// dK, dV of one key cube.  2 waves; wave w owns keys 32w .. 32w + 31 and all
// 64 queries of each query tile that selected this key cube:
//   S  = Q K^T,  dP = dOf V^T      (m = queries, n = keys, k = d)
//   P = exp(s S - lse), dS = P (dP - Delta)
//   dV^T += dOf^T P,  dK^T += Q^T dS  (m = d, n = keys, k = queries)
template <int D>
__global__ __launch_bounds__(128, 1) void fine_bwd_dkdv_kernel(
    const bf16* __restrict__ qp, const bf16* __restrict__ kp, const bf16* __restrict__ vp,
    const bf16* __restrict__ qt, const bf16* __restrict__ dofp, const bf16* __restrict__ doft,
    const float* __restrict__ lse_f, const float* __restrict__ delta,
    const int32_t* __restrict__ tr_offs, const int32_t* __restrict__ tr_ids,
    const float* __restrict__ dkc, const float* __restrict__ dvc,
    int nh, int nc, int Hg, int Wg, float scale,
    bf16* __restrict__ dk, bf16* __restrict__ dv) {
  constexpr int KS = D / 16, KCH = D / 8, MD = D / 32;
  __shared__ __align__(16) u32x4 q_lds[64 * KCH];
  __shared__ __align__(16) u32x4 do_lds[64 * KCH];
  __shared__ __align__(16) u32x4 qt_lds[D * 8];
  __shared__ __align__(16) u32x4 dot_lds[D * 8];
  __shared__ float lse_s[64], del_s[64];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ql = lane & 31, hf = lane >> 5;
  const int blk = blockIdx.x;  // (b*nh + h)*nc + key cube
  const int bh = blk / nc, j = blk - bh * nc;
  const int64_t N = (int64_t)nc * 64;
  const int64_t bh_tiles = (int64_t)bh * nc;
  const float scale_log2 = scale * kLog2e;

  // K and V rows of this wave's keys as B operands: lane (key, hf) holds
  // d = (D/2) hf + 8 s .. +8.
  bf16x8 kB[KS], vB[KS];
  {
    const int64_t row = (bh_tiles + j) * 64 + 32 * wave + ql;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kB[s] = *reinterpret_cast<const bf16x8*>(kp + row * D + (D / 2) * hf + 8 * s);
      vB[s] = *reinterpret_cast<const bf16x8*>(vp + row * D + (D / 2) * hf + 8 * s);
    }
  }
  f32x16 dka[MD], dva[MD];
#pragma unroll
  for (int m = 0; m < MD; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dka[m][r] = 0.f; dva[m][r] = 0.f; }

  const int e0 = tr_offs[blk], e1 = tr_offs[blk + 1];
  for (int e = e0; e < e1; ++e) {
    const int c = tr_ids[e];
    const int64_t t = (bh_tiles + c) * 64;
    __syncthreads();
    stage_nat<D, 128>(qp + t * D, q_lds, tid);
    stage_nat<D, 128>(dofp + t * D, do_lds, tid);
    stage_tr<D, 128>(qt + t * D, qt_lds, tid);
    stage_tr<D, 128>(doft + t * D, dot_lds, tid);
    if (tid < 64) lse_s[tid] = lse_f[(int64_t)bh * N + (int64_t)c * 64 + tid] * kLog2e;
    else del_s[tid - 64] = delta[(int64_t)bh * N + (int64_t)c * 64 + tid - 64];
    __syncthreads();

    bf16x8 pB[2][2], dsB[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x16 sa, da;
#pragma unroll
      for (int r = 0; r < 16; ++r) { sa[r] = 0.f; da[r] = 0.f; }
      const int qrow = 32 * mb + ql;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int chk = (KS * hf + s) ^ swz_row<D>(qrow);
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&q_lds[qrow * KCH + chk]);
        const bf16x8 oa = *reinterpret_cast<const bf16x8*>(&do_lds[qrow * KCH + chk]);
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kB[s], sa, 0, 0, 0);
        da = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vB[s], da, 0, 0, 0);
      }
      // this lane: key column ql, query rows 32mb + 8(r/4) + 4hf + r%4
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) {
          const int r = 8 * g + e8;
          const int q = 32 * mb + 8 * (r >> 2) + 4 * hf + (r & 3);
          const float p = __builtin_amdgcn_exp2f(fmaf(sa[r], scale_log2, -lse_s[q]));
          pB[mb][g][e8] = (bf16)p;
          dsB[mb][g][e8] = (bf16)(p * (da[r] - del_s[q]));
        }
    }
    // dV^T += dOf^T P,  dK^T += Q^T dS : k-steps (mb, g) over 64 queries
#pragma unroll
    for (int m = 0; m < MD; ++m) {
      const int row = 32 * m + ql;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int chk = (2 * (2 * mb + g) + hf) ^ swz_t(row);
          const bf16x8 oa = *reinterpret_cast<const bf16x8*>(&dot_lds[row * 8 + chk]);
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&qt_lds[row * 8 + chk]);
          dva[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, pB[mb][g], dva[m], 0, 0, 0);
          dka[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, dsB[mb][g], dka[m], 0, 0, 0);
        }
    }
  }

  // raster rows of this wave's keys, coarse share (mean adjoint) added
  const int slot = 32 * wave + ql;
  const int b = bh / nh, h = bh - b * nh;
  const int tok = raster_tok(j, slot, Hg, Wg);
  const int64_t gidx = ((int64_t)b * N + tok) * nh + h;
  const float* kcr = dkc + (bh_tiles + j) * D;
  const float* vcr = dvc + (bh_tiles + j) * D;
#pragma unroll
  for (int m = 0; m < MD; ++m)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = 32 * m + 8 * rg + 4 * hf;
      const f32x4 ck = *reinterpret_cast<const f32x4*>(kcr + d0);
      const f32x4 cv = *reinterpret_cast<const f32x4*>(vcr + d0);
      bf16x4 ok, ov;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ok[i] = (bf16)fmaf(scale, dka[m][4 * rg + i], ck[i] * (1.0f / kCubeTokens));
        ov[i] = (bf16)(dva[m][4 * rg + i] + cv[i] * (1.0f / kCubeTokens));
      }
      *reinterpret_cast<bf16x4*>(dk + gidx * D + d0) = ok;
      *reinterpret_cast<bf16x4*>(dv + gidx * D + d0) = ov;
    }
}

// dQ of one query cube.  2 waves; wave w owns queries 32w .. 32w + 31:
//   S^T = K Q^T, dP^T = V dOf^T    (m = keys, n = queries, k = d)
//   dS^T = P^T (dP^T - Delta)
//   dQ = sum over tiles t of  dS_t (K_t - kc_t)  +  s_t kc_t,
//        s_t = sum of dS over the keys of tile t (fp32)
// The first term runs on MFMA with K^T tiles centred on their cube mean
// kc_t (kt holds K - kc); the second is an fp32 vector update.  Because the
// exact dS sums to zero over a row, sum_t s_t c adds nothing for any fixed
// vector c; taking c = kc of the row's first tile removes the rounding
// residue of sum_t s_t along the keys' large shared component, which would
// otherwise dominate dQ when the selected cubes share a mean.
template <int D>
__global__ __launch_bounds__(128, 1) void fine_bwd_dq_kernel(
    const bf16* __restrict__ qp, const bf16* __restrict__ kp, const bf16* __restrict__ vp,
    const bf16* __restrict__ kt, const bf16* __restrict__ dofp,
    const float* __restrict__ lse_f, const float* __restrict__ delta,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ ids, int topk,
    const float* __restrict__ dqc, const float* __restrict__ kc_mean,
    int nh, int nc, int Hg, int Wg, float scale, bf16* __restrict__ dq) {
  constexpr int KS = D / 16, KCH = D / 8, MD = D / 32;
  __shared__ __align__(16) u32x4 k_lds[64 * KCH];
  __shared__ __align__(16) u32x4 v_lds[64 * KCH];
  __shared__ __align__(16) u32x4 kt_lds[D * 8];
  __shared__ __align__(16) float kc_s[D];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ql = lane & 31, hf = lane >> 5;
  const int blk = blockIdx.x;  // (b*nh + h)*nc + query cube
  const int bh = blk / nc, c = blk - bh * nc;
  const int64_t N = (int64_t)nc * 64;
  const int64_t bh_tiles = (int64_t)bh * nc;
  const float scale_log2 = scale * kLog2e;
  int start, n;
  if (offs) { start = offs[blk]; n = offs[blk + 1] - start; }
  else { start = blk * topk; n = topk; }

  const int slot = 32 * wave + ql;
  bf16x8 qB[KS], oB[KS];
  {
    const int64_t row = (bh_tiles + c) * 64 + slot;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qB[s] = *reinterpret_cast<const bf16x8*>(qp + row * D + (D / 2) * hf + 8 * s);
      oB[s] = *reinterpret_cast<const bf16x8*>(dofp + row * D + (D / 2) * hf + 8 * s);
    }
  }
  const float lse2 = lse_f[(int64_t)bh * N + (int64_t)c * 64 + slot] * kLog2e;
  const float del = delta[(int64_t)bh * N + (int64_t)c * 64 + slot];
  f32x16 dqa[MD], cor[MD];
#pragma unroll
  for (int m = 0; m < MD; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dqa[m][r] = 0.f; cor[m][r] = 0.f; }
  float ssum = 0.f;

  for (int it = 0; it < n; ++it) {
    const int kc = ids[start + it];
    const int64_t t = (bh_tiles + kc) * 64;
    __syncthreads();
    stage_nat<D, 128>(kp + t * D, k_lds, tid);
    stage_nat<D, 128>(vp + t * D, v_lds, tid);
    stage_tr<D, 128>(kt + t * D, kt_lds, tid);
    if (tid < D) kc_s[tid] = kc_mean[(bh_tiles + kc) * D + tid];
    __syncthreads();
    bf16x8 dsB[2][2];
    float st = 0.f;  // sum of this lane's dS over its keys of the tile
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x16 sa, da;
#pragma unroll
      for (int r = 0; r < 16; ++r) { sa[r] = 0.f; da[r] = 0.f; }
      const int krow = 32 * mb + ql;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int chk = (KS * hf + s) ^ swz_row<D>(krow);
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&k_lds[krow * KCH + chk]);
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(&v_lds[krow * KCH + chk]);
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qB[s], sa, 0, 0, 0);
        da = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, oB[s], da, 0, 0, 0);
      }
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) {
          const int r = 8 * g + e8;
          const float p = __builtin_amdgcn_exp2f(fmaf(sa[r], scale_log2, -lse2));
          const float ds = p * (da[r] - del);
          st += ds;
          dsB[mb][g][e8] = (bf16)ds;
        }
    }
    st += swap_halves(st);
    ssum += st;
#pragma unroll
    for (int m = 0; m < MD; ++m)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(&kc_s[32 * m + 8 * rg + 4 * hf]);
#pragma unroll
        for (int i = 0; i < 4; ++i) cor[m][4 * rg + i] = fmaf(st, kv[i], cor[m][4 * rg + i]);
      }
#pragma unroll
    for (int m = 0; m < MD; ++m) {
      const int row = 32 * m + ql;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int chk = (2 * (2 * mb + g) + hf) ^ swz_t(row);
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&kt_lds[row * 8 + chk]);
          dqa[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, dsB[mb][g], dqa[m], 0, 0, 0);
        }
    }
  }

  const int b = bh / nh, h = bh - b * nh;
  const int tok = raster_tok(c, slot, Hg, Wg);
  const int64_t gidx = ((int64_t)b * N + tok) * nh + h;
  const float* qcr = dqc + (bh_tiles + c) * D;
  const float* c0 = kc_mean + (bh_tiles + (n > 0 ? ids[start] : 0)) * D;
#pragma unroll
  for (int m = 0; m < MD; ++m)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = 32 * m + 8 * rg + 4 * hf;
      const f32x4 cq = *reinterpret_cast<const f32x4*>(qcr + d0);
      const f32x4 cc = *reinterpret_cast<const f32x4*>(c0 + d0);
      bf16x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * rg + i;
        const float fine = dqa[m][r] + (cor[m][r] - ssum * cc[i]);
        o[i] = (bf16)fmaf(scale, fine, cq[i] * (1.0f / kCubeTokens));
      }
      *reinterpret_cast<bf16x4*>(dq + gidx * D + d0) = o;
    }
}

template <bool TA, bool TB>
hipError_t gemm(const float* A, int lda, int64_t sA, const float* B, int ldb, int64_t sB,
                float* C, int ldc, int64_t sC, int M, int N, int K, float alpha, int batch,
                hipStream_t st) {
  dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64), (unsigned)batch);
  gemm_f32_kernel<TA, TB><<<grid, 256, 0, st>>>(A, lda, sA, B, ldb, sB, C, ldc, sC, M, N, K, alpha);
  return hipGetLastError();
}

template <int D>
hipError_t launch_backward_d(const BackwardArgs& a, hipStream_t st) {
  const int nc = (a.T / 4) * (a.H / 4) * (a.W / 4);
  const int BH = a.B * a.heads;
  const float scale = 1.0f / sqrtf((float)D);
  hipError_t e;
#define VSA_TRY(x) do { e = (x); if (e != hipSuccess) return e; } while (0)
  bwd_prep_kernel<D><<<(unsigned)(a.B * nc * a.heads), 256, 0, st>>>(
      (const bf16*)a.dout, (const bf16*)a.gc, (const bf16*)a.gf, a.of, a.oc, a.heads, a.T, a.H, a.W,
      (float*)a.dgc, (float*)a.dgf, a.delta, (bf16*)a.dofp, (bf16*)a.doft, a.doc, a.deltac);
  VSA_TRY(hipGetLastError());
  // coarse backward on the cube means
  const int64_t sq = (int64_t)nc * D, ss = (int64_t)nc * nc;
  VSA_TRY((gemm<false, true>(a.qc, D, sq, a.kc, D, sq, a.S, nc, ss, nc, nc, D, scale, BH, st)));
  VSA_TRY((gemm<false, true>(a.doc, D, sq, a.vc, D, sq, a.dP, nc, ss, nc, nc, D, 1.0f, BH, st)));
  const int64_t rows = (int64_t)BH * nc;
  coarse_softmax_grad_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, st>>>(a.S, a.dP, a.lse_c, a.deltac, nc, rows);
  VSA_TRY(hipGetLastError());
  VSA_TRY((gemm<false, false>(a.dP, nc, ss, a.kc, D, sq, a.dqc, D, sq, nc, D, nc, scale, BH, st)));
  VSA_TRY((gemm<true, false>(a.dP, nc, ss, a.qc, D, sq, a.dkc, D, sq, nc, D, nc, scale, BH, st)));
  VSA_TRY((gemm<true, false>(a.S, nc, ss, a.doc, D, sq, a.dvc, D, sq, nc, D, nc, 1.0f, BH, st)));
  // transposed selection
  transpose_lists_kernel<<<(unsigned)BH, 256, sizeof(int32_t) * (2 * nc + 1), st>>>(
      a.offs, a.ids, a.topk, nc, a.tr_offs, a.tr_ids);
  VSA_TRY(hipGetLastError());
  const unsigned grid = (unsigned)(BH * nc);
  fine_bwd_dkdv_kernel<D><<<grid, 128, 0, st>>>(
      (const bf16*)a.qp, (const bf16*)a.kp, (const bf16*)a.vp, (const bf16*)a.qt,
      (const bf16*)a.dofp, (const bf16*)a.doft, a.lse_f, a.delta, a.tr_offs, a.tr_ids,
      a.dkc, a.dvc, a.heads, nc, a.H, a.W, scale, (bf16*)a.dk, (bf16*)a.dv);
  VSA_TRY(hipGetLastError());
  fine_bwd_dq_kernel<D><<<grid, 128, 0, st>>>(
      (const bf16*)a.qp, (const bf16*)a.kp, (const bf16*)a.vp, (const bf16*)a.kt,
      (const bf16*)a.dofp, a.lse_f, a.delta, a.offs, a.ids, a.topk, a.dqc, a.kc,
      a.heads, nc, a.H, a.W, scale, (bf16*)a.dq);
  VSA_TRY(hipGetLastError());
#undef VSA_TRY
  return hipSuccess;
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, hipStream_t st) {
  return a.D == 128 ? launch_backward_d<128>(a, st) : launch_backward_d<64>(a, st);
}

}  // namespace vsa
