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
//                   Delta = dOf.O_fine, dOf = g_f dO (bf16 cube tile),
//                   dOc = sum over the cube of g_c dO and Delta_c = dOc.Oc
//   gemm_f32 / coarse_softmax_grad
//                   coarse backward on the means: S, dP by fp32 MFMA GEMMs
//                   (one launch), P = exp(S - lse_c), dS = P (dP - Delta_c),
//                   then dQc = s dS Kc, and dKc = s dS^T Qc with
//                   dVc = P^T dOc (one launch)
//   transpose_scatter / transpose_rank
//                   for every key cube, the ascending list of query cubes
//                   that selected it (counting sort per (b, h), then a rank
//                   sort of each list, one wave per list)
//   fine_bwd_dkdv   key-stationary: one workgroup per key cube accumulates
//                   dK and dV over the query cubes that selected it, and
//                   (bf16) stores each pair's dS tile
//   fine_bwd_dq     query-stationary: one workgroup per query cube
//                   accumulates dQ over its selected key cubes (bf16: from
//                   the stored dS tiles, one product per pair)
// The last two write raster-order gradients with the coarse share added.
// Both stream their per-pair tiles (Q and dOf, resp. K and the 8 KB dS
// tile, or K and V for fp32; 16 KB each at D = 128, natural row-major
// layout) with global->LDS copies, double buffered, and take every
// transposed operand from transposing LDS reads.
// Each wave raises its issue priority for its two MFMA bursts per tile
// (s_setprio 1, back to 0 for the softmax arithmetic), so a SIMD's matrix
// unit is fed first while the other resident wave runs its VALU work; the
// order of every wave's own arithmetic, hence the result, is unchanged.
#include <climits>

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
// Eight consecutive elements of a bf16 or fp32 row as floats, and back.
__device__ __forceinline__ void load8(const bf16* p, float (&x)[8]) {
  const u32x4 raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  bf16 v[8];
  __builtin_memcpy(v, &raw, 16);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
#pragma unroll
  for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
}
__device__ __forceinline__ void store8(bf16* p, const bf16 (&v)[8]) {
  u32x4 packed;
  __builtin_memcpy(&packed, v, 16);
  *reinterpret_cast<u32x4*>(p) = packed;
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  *(reinterpret_cast<f32x4*>(p) + 1) = f32x4{v[4], v[5], v[6], v[7]};
}

// T: element type of dO, the gates and the dOf tile (bf16 or fp32).
template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_prep_kernel(
    const T* __restrict__ dout, const T* __restrict__ gc, const T* __restrict__ gf,
    const float* __restrict__ of, const float* __restrict__ oc, int nh, int Tg, int Hg, int Wg,
    float* __restrict__ dgc, float* __restrict__ dgf, float* __restrict__ delta,
    T* __restrict__ dofp, float* __restrict__ doc, float* __restrict__ deltac) {
  constexpr int EPC = 8;
  constexpr int CPR = D / EPC;
  constexpr int RPP = 256 / CPR;
  constexpr int PASSES = kCubeTokens / RPP;
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

  // All passes' loads first, so that they are in flight together (the
  // compiler keeps each pass's loads behind the previous pass's stores).
  // dO and O_fine are read once in the backward: non-temporal loads.
  float gvs[PASSES][EPC];
  f32x4 o0s[PASSES], o1s[PASSES];
  float gcv[PASSES], gfv[PASSES];
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int s = tid / CPR + ps * RPP;
    const int64_t gidx = ((int64_t)b * N + raster_tok(c, s, Hg, Wg)) * nh + h;
    load8(dout + gidx * D + ch * EPC, gvs[ps]);
    gcv[ps] = (float)gc[gidx];
    gfv[ps] = (float)gf[gidx];
    const f32x4* op = reinterpret_cast<const f32x4*>(of + ((int64_t)bh * N + (int64_t)c * 64 + s) * D + ch * EPC);
    o0s[ps] = __builtin_nontemporal_load(op);
    o1s[ps] = __builtin_nontemporal_load(op + 1);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int s = tid / CPR + ps * RPP;
    const int tok = raster_tok(c, s, Hg, Wg);
    const int64_t gidx = ((int64_t)b * N + tok) * nh + h;
    const float gcs = gcv[ps], gfs = gfv[ps];
    const f32x4 o0 = o0s[ps], o1 = o1s[ps];
    // pc, pf: dO.Oc and dO.O_fine (the gate gradients, fp32).  pd is
    // Delta = dOf.O_fine taken with dOf rounded to the element type exactly
    // as the fine kernels use it, so that sum_j P_ij dP_ij = Delta_i holds
    // to fp32 accuracy and dS sums to zero over each row.
    float pc = 0.f, pf = 0.f, pd = 0.f;
    T dv[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const float g = gvs[ps][e];
      const float ofe = e < 4 ? o0[e] : o1[e - 4];
      pc = fmaf(g, ocv[e], pc);
      pf = fmaf(g, ofe, pf);
      acc[e] = fmaf(gcs, g, acc[e]);
      dv[e] = from_f32<T>(gfs * g);
      pd = fmaf(to_f32(dv[e]), ofe, pd);
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
    store8(dofp + tile + (int64_t)s * D + ch * EPC, dv);
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
  __syncthreads();
  if (tid < 64) {  // Delta_c = dOc . Oc: one wave folds the D products
    float t = 0.f;
#pragma unroll
    for (int d = tid; d < D; d += 64) t += dsum[d];
    t = wave_sum(t);
    if (tid == 0) deltac[(int64_t)bh * nc + c] = t;
  }
}

// ---------------------------------------------------------------- coarse
typedef float f32x4v __attribute__((ext_vector_type(4)));

// Up to two products of one shape per launch (operands of product p in
// GemmPair slot p; blockIdx.z = p * batch + z).
struct GemmPair {
  const float* A[2];
  const float* B[2];
  float* C[2];
  float alpha[2];
};

// C[z] = alpha * op(A[z]) * op(B[z]) for z < batch, fp32, row-major.
// op(A) is M x K (TA: A stored K x M); op(B) is K x N (TB: B stored N x K).
// 64 x 64 output tile per workgroup, v_mfma_f32_16x16x4f32, each wave owns a
// 32 x 32 quarter.  K runs in 32-deep chunks staged through LDS; the next
// chunk's loads (8 + 8 floats per thread, consecutive threads on the
// contiguous dimension of each operand) are issued before the current chunk
// is multiplied, so their latency overlaps the MFMAs.
template <bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    GemmPair g, int batch, int lda, int64_t sA, int ldb, int64_t sB, int ldc, int64_t sC, int M, int N,
    int K) {
  constexpr int KC = 32;
  __shared__ float As[KC][64 + 4];
  __shared__ float Bs[KC][64 + 4];
  const int pr = (int)blockIdx.z >= batch ? 1 : 0;
  const int z = (int)blockIdx.z - pr * batch;
  const float* __restrict__ A = g.A[pr] + z * sA;
  const float* __restrict__ B = g.B[pr] + z * sB;
  float* __restrict__ C = g.C[pr] + z * sC;
  const float alpha = g.alpha[pr];
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, lg = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  f32x4v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4v{0.f, 0.f, 0.f, 0.f};

  // element e of this thread's share of a chunk: (k, m) of A and (k, n) of B
  auto a_km = [&](int e, int& kk, int& mm) {
    const int i = tid + 256 * e;
    if (TA) { kk = i / 64; mm = i % 64; } else { mm = i / KC; kk = i % KC; }
  };
  auto b_kn = [&](int e, int& kk, int& nn) {
    const int i = tid + 256 * e;
    if (TB) { nn = i / KC; kk = i % KC; } else { kk = i / 64; nn = i % 64; }
  };
  float ra[8], rb[8];
  auto load_chunk = [&](int k0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int kk, mm, nn, kb;
      a_km(e, kk, mm);
      const int gm = m0 + mm, gk = k0 + kk;
      ra[e] = (gm < M && gk < K) ? (TA ? A[(int64_t)gk * lda + gm] : A[(int64_t)gm * lda + gk]) : 0.f;
      b_kn(e, kb, nn);
      const int gn = n0 + nn, gk2 = k0 + kb;
      rb[e] = (gn < N && gk2 < K) ? (TB ? B[(int64_t)gn * ldb + gk2] : B[(int64_t)gk2 * ldb + gn]) : 0.f;
    }
  };
  load_chunk(0);
  for (int k0 = 0; k0 < K; k0 += KC) {
    __syncthreads();  // the previous chunk's reads are done
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int kk, mm, nn, kb;
      a_km(e, kk, mm);
      As[kk][mm] = ra[e];
      b_kn(e, kb, nn);
      Bs[kb][nn] = rb[e];
    }
    __syncthreads();
    if (k0 + KC < K) load_chunk(k0 + KC);
#pragma unroll
    for (int t = 0; t < KC / 4; ++t) {
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
//
// Exclusive prefix sum of in[0..n) into out[0..n] (out[n] = total) by the
// 256 threads of a workgroup: thread t owns in[t L .. t L + L).  Ends with
// a barrier.
__device__ void block_exclusive_scan(const int32_t* in, int n, int32_t* out, int32_t* wsum) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int L = (n + 255) / 256;
  const int lo = min(tid * L, n), hi = min(lo + L, n);
  int own = 0;
  for (int j = lo; j < hi; ++j) own += in[j];
  int incl = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int run = incl - own;
  for (int w = 0; w < wave; ++w) run += wsum[w];
  for (int j = lo; j < hi; ++j) { out[j] = run; run += in[j]; }
  if (tid == 255) out[n] = run;
  __syncthreads();
}

// transpose_scatter: one workgroup per (b, h): counts (LDS atomics), an
// exclusive scan into tr_offs, then a scatter of the query cube ids into
// `tmp`, each list in arbitrary order, and (tmp_pos non-null) of each
// entry's index in `ids` into tmp_pos at the same slot.  It also writes tr_order, the key
// cubes of (b, h) by list length, longest first: the dK/dV kernel takes
// them in that order, so that the longest lists start first and the
// workgroups running together have lists of similar length (their sweeps
// over the query cubes stay in step, which helps L2 reuse).  The order
// among equal lengths is arbitrary; results do not depend on it.
__global__ __launch_bounds__(256) void transpose_scatter_kernel(
    const int32_t* __restrict__ offs, const int32_t* __restrict__ ids, int topk, int64_t n_ids,
    int nc, int32_t* __restrict__ tr_offs, int32_t* __restrict__ tr_order, int32_t* __restrict__ tmp,
    int32_t* __restrict__ tmp_pos) {
  // LDS: cnt [nc] (counts, then cursors), start [nc + 1], hist [nc + 1],
  // hpos [nc + 2]
  extern __shared__ int32_t cnt[];
  __shared__ int32_t wsum[4];
  int32_t* start = cnt + nc;
  int32_t* hist = start + nc + 1;
  int32_t* hpos = hist + nc + 1;
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)bh * nc;
  // Entries of this (b, h): [base, base + total), clamped to the id array;
  // every position written below stays inside it whatever the offsets hold.
  const int64_t base = offs ? min(max((int64_t)offs[r0], (int64_t)0), n_ids) : r0 * topk;
  const int total = (int)((offs ? min(max((int64_t)offs[r0 + nc], base), n_ids)
                                : (r0 + nc) * topk) - base);
  for (int j = tid; j < nc; j += 256) cnt[j] = 0;
  for (int v = tid; v <= nc; v += 256) hist[v] = 0;
  __syncthreads();
  // Entries are read kBatch at a time, so that their loads are in flight
  // together rather than one memory round trip per entry.
  constexpr int kBatch = 8;
  for (int e0 = tid; e0 < total; e0 += 256 * kBatch) {
    int jj[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) jj[u] = e0 + 256 * u < total ? ids[base + e0 + 256 * u] : -1;
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (jj[u] >= 0 && jj[u] < nc) atomicAdd(&cnt[jj[u]], 1);
  }
  __syncthreads();
  block_exclusive_scan(cnt, nc, start, wsum);
  for (int j = tid; j <= nc; j += 256) tr_offs[r0 + j] = base + start[j];
  // key cubes by list length, longest first (a query cube picks a key cube
  // at most once, so lengths are at most nc)
  for (int j = tid; j < nc; j += 256) atomicAdd(&hist[min(cnt[j], nc)], 1);
  __syncthreads();
  block_exclusive_scan(hist, nc + 1, hpos, wsum);
  for (int v = tid; v <= nc; v += 256) hist[v] = 0;  // cursors per length
  __syncthreads();
  for (int j = tid; j < nc; j += 256) {
    const int v = min(cnt[j], nc);
    tr_order[r0 + (nc - hpos[v + 1]) + atomicAdd(&hist[v], 1)] = j;
  }
  __syncthreads();
  for (int j = tid; j < nc; j += 256) cnt[j] = start[j];  // fill cursors
  __syncthreads();
  for (int c = tid; c < nc; c += 256) {
    int64_t e0;
    int len;
    list_range(offs, r0 + c, topk, n_ids, &e0, &len);
    const int64_t e1 = e0 + len;
    for (int64_t e = e0; e < e1; e += kBatch) {
      int jj[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) jj[u] = e + u < e1 ? ids[e + u] : -1;
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (cube_ok(jj[u], nc)) {
          // rows of well-formed offsets tile [base, base + total) exactly;
          // others may not, and what would not fit is dropped
          const int pos = atomicAdd(&cnt[jj[u]], 1);
          if (pos < total) {
            tmp[base + pos] = c;
            if (tmp_pos) tmp_pos[base + pos] = (int32_t)(e + u);
          }
        }
    }
  }
}

// transpose_rank: one wave per list r < n_lists, sorting it by rank: every
// lane counts the entries that precede its own, smaller values first and
// equal values by position (a query cube that lists a key cube twice
// appears twice), through readlane broadcasts.  Ranks are therefore
// distinct and every slot of the list is written.  With tr_pos, each
// entry's index in `ids` moves along with it.
__global__ __launch_bounds__(256) void transpose_rank_kernel(
    const int32_t* __restrict__ tr_offs, const int32_t* __restrict__ tmp,
    const int32_t* __restrict__ tmp_pos, int64_t n_lists, int64_t n_ids,
    int32_t* __restrict__ tr_ids, int32_t* __restrict__ tr_pos) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n_lists) return;
  int64_t s0;
  int n;
  list_range(tr_offs, r, 0, n_ids, &s0, &n);
  const int32_t* lst = tmp + s0;
  for (int c0 = 0; c0 < n; c0 += 64) {
    const int idx = c0 + lane;
    const int v = idx < n ? lst[idx] : INT_MAX;
    int rank = 0;
    for (int k0 = 0; k0 < n; k0 += 64) {
      const int u = k0 + lane < n ? lst[k0 + lane] : INT_MAX;
      const int m = min(64, n - k0);
      for (int i = 0; i < m; ++i) {
        const int w = __builtin_amdgcn_readlane(u, i);
        rank += w < v || (w == v && k0 + i < idx);
      }
    }
    if (idx < n) {
      tr_ids[s0 + rank] = v;
      if (tr_pos) tr_pos[s0 + rank] = tmp_pos[s0 + idx];
    }
  }
}

// ---------------------------------------------------------------- fine
// dK, dV of one key cube.  4 waves; wave w: key half kh = w & 1 (keys
// 32kh .. +32), query half qh = w >> 1 of every query tile that selected
// this key cube.  Per query tile:
//   S  = Q K^T,  dP = dOf V^T        (m = 32 queries, n = 32 keys, k = d)
//   P = exp(s S - lse), dS = P (dP - Delta)
// then the two waves of a key half swap half of their results through LDS
// (the qh = 0 wave hands over dS, the qh = 1 wave P), and over all 64
// queries (m = d, n = keys, k = queries)
//   qh = 0:  dV^T += dOf^T P          qh = 1:  dK^T += Q^T dS
// with dOf^T and Q^T read transposed from the natural tiles.
template <int D>
__global__ __launch_bounds__(256, 2) void fine_bwd_dkdv_kernel(
    const bf16* __restrict__ qp, const bf16* __restrict__ kp, const bf16* __restrict__ vp,
    const bf16* __restrict__ dofp, const float* __restrict__ lse_f, const float* __restrict__ delta,
    const int32_t* __restrict__ tr_offs, const int32_t* __restrict__ tr_order,
    const int32_t* __restrict__ tr_ids, const int32_t* __restrict__ tr_pos, int64_t n_ids,
    const float* __restrict__ dkc, const float* __restrict__ dvc, int nh, int nc, int Hg, int Wg,
    float scale, int n_logical, bf16* __restrict__ dk, bf16* __restrict__ dv, bf16* __restrict__ ds) {
  constexpr int KS = D / 16, MD = D / 32, TILE_CH = 64 * D / 8;
  // Tile parity buffers: separate arrays picked at run time, so that the
  // compiler adds no waits of its own for the global->LDS copies.
  __shared__ __align__(256) u32x4 q_lds0[TILE_CH];
  __shared__ __align__(256) u32x4 q_lds1[TILE_CH];
  __shared__ __align__(256) u32x4 o_lds0[TILE_CH];
  __shared__ __align__(256) u32x4 o_lds1[TILE_CH];
  __shared__ __align__(16) float ld_s0[128];  // lse (64 queries), then Delta (64)
  __shared__ __align__(16) float ld_s1[128];
  __shared__ __align__(16) bf16x8 xch[4][2][64];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ql = lane & 31, hf = lane >> 5;
  const int kh = wave & 1, qh = wave >> 1;
  // Logical block (b*nh + h)*nc + rank of the key cube by list length,
  // numbered XCD-contiguously (hardware block i runs on XCD i % 8): each XCD
  // works through whole heads, longest lists first, and keeps one head's
  // Q and dO tiles in its own L2.  Padding blocks exit at once.
  const int per = (n_logical + 7) >> 3;
  const int blk = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (blk >= n_logical) return;
  const int bh = blk / nc;
  const int64_t N = (int64_t)nc * 64;
  const int64_t bh_tiles = (int64_t)bh * nc;
  const int j = tr_order[blk];
  const float scale_log2 = scale * kLog2e;

  // K and V rows of this wave's keys as B operands: lane (key, hf) holds
  // d = (D/2) hf + 8 s .. +8.
  bf16x8 kB[KS], vB[KS];
  {
    const int64_t row = (bh_tiles + j) * 64 + 32 * kh + ql;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kB[s] = *reinterpret_cast<const bf16x8*>(kp + row * D + (D / 2) * hf + 8 * s);
      vB[s] = *reinterpret_cast<const bf16x8*>(vp + row * D + (D / 2) * hf + 8 * s);
    }
  }
  f32x16 acc[MD];
#pragma unroll
  for (int m = 0; m < MD; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[m][r] = 0.f;

  const uint32_t tr_lo = tr_offset<D>(lane, 0), tr_hi = tr_offset<D>(lane, 1);
  int64_t e0;
  int n;
  list_range(tr_offs, bh_tiles + j, 0, n_ids, &e0, &n);
  auto copy_tile = [&](int c, int buf) {
    c = cube_or_0(c, nc);  // the library's own transposed lists always pass
    const int64_t t = (bh_tiles + c) * 64;
    dma_tile<D>(qp + t * D, buf ? q_lds1 : q_lds0, wave, lane);
    dma_tile<D>(dofp + t * D, buf ? o_lds1 : o_lds0, wave, lane);
    if (wave == 0 && lane < 32) {  // 16 lanes of lse, 16 of Delta
      const int64_t tok = (int64_t)bh * N + (int64_t)c * 64 + 4 * (lane & 15);
      copy16_to_lds(lane < 16 ? lse_f + tok : delta + tok, buf ? ld_s1 : ld_s0);
    }
  };
  if (n > 0) copy_tile(tr_ids[e0], 0);

  for (int it = 0; it < n; ++it) {
    const int buf = it & 1;
    wait_vmcnt<0>();   // this wave's copies of tile `it` have landed
    __syncthreads();   // all copies visible; buffer buf^1 and xch free
    if (it + 1 < n) copy_tile(tr_ids[e0 + it + 1], buf ^ 1);
    const u32x4* qb = buf ? q_lds1 : q_lds0;
    const u32x4* ob = buf ? o_lds1 : o_lds0;
    const float* ls = buf ? ld_s1 : ld_s0;

    bf16x8 qa[KS], oa[KS];
    const int qrow = 32 * qh + ql;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qa[s] = tile_row8<D>(qb, qrow, KS * hf + s);
      oa[s] = tile_row8<D>(ob, qrow, KS * hf + s);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x16 sa, da;
#pragma unroll
    for (int r = 0; r < 16; ++r) { sa[r] = 0.f; da[r] = 0.f; }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s], kB[s], sa, 0, 0, 0);
      da = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[s], vB[s], da, 0, 0, 0);
    }
    // Q^T (dK wave) or dOf^T (dV wave) operands of column block 0, read
    // while the MFMAs above run; blocks m > 0 follow the MFMAs of m - 1.
    const uint32_t xbase = lds_addr(qh ? qb : ob);
    bf16x8 xa[4];
    tile_tr8_asm<D, 4>(xa, xbase + tr_lo, xbase + tr_hi);
    __builtin_amdgcn_s_setprio(0);
    // this lane: key column ql, query rows 32qh + 8(r/4) + 4hf + r%4
    bf16x8 pB[2], dsB[2];
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int q0 = 32 * qh + 8 * rg + 4 * hf;
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(ls + q0);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(ls + 64 + q0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * rg + i;
        const float p = __builtin_amdgcn_exp2f(fmaf(sa[r], scale_log2, -l4[i] * kLog2e));
        pB[r >> 3][r & 7] = (bf16)p;
        dsB[r >> 3][r & 7] = (bf16)(p * (da[r] - d4[i]));
      }
    }
    // this wave's dS block, kept for the dQ pass: the pair's 64 x 64 tile
    // (entry tr_pos of the key lists) as dS^T, rows = keys, row-major; this
    // lane's key row, queries 32qh + 8a + 4hf .. +4 per 8-byte store
    {
      const int64_t ent = tr_pos[e0 + it];
      if ((uint64_t)ent < (uint64_t)n_ids) {
        bf16* drow = ds + ent * 4096 + (int64_t)(32 * kh + ql) * 64 + 32 * qh + 4 * hf;
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const bf16x8& src = dsB[a4 >> 1];
          const int e = 4 * (a4 & 1);
          *reinterpret_cast<bf16x4*>(drow + 8 * a4) = bf16x4{src[e], src[e + 1], src[e + 2], src[e + 3]};
        }
      }
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) xch[wave][g][lane] = qh ? pB[g] : dsB[g];
    lds_barrier();
    bf16x8 bq0[2], bq1[2];  // B operands for queries 0..31 and 32..63
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const bf16x8 other = xch[wave ^ 2][g][lane];
      bq0[g] = qh ? other : pB[g];
      bq1[g] = qh ? dsB[g] : other;
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int m = 0; m < MD; ++m) {
      if (m > 0) tile_tr8_asm<D, 4>(xa, (xbase + tr_lo) ^ (m << 6), (xbase + tr_hi) ^ (m << 6));
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[t], t < 2 ? bq0[t] : bq1[t - 2], acc[m], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // raster rows of this wave's keys, coarse share (mean adjoint) added
  const int slot = 32 * kh + ql;
  const int b = bh / nh, h = bh - b * nh;
  const int tok = raster_tok(j, slot, Hg, Wg);
  const int64_t gidx = ((int64_t)b * N + tok) * nh + h;
  const float* crow = (qh ? dkc : dvc) + (bh_tiles + j) * D;
  bf16* orow = (qh ? dk : dv) + gidx * D;
  const float mul = qh ? scale : 1.0f;
#pragma unroll
  for (int m = 0; m < MD; ++m)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = 32 * m + 8 * rg + 4 * hf;
      const f32x4 cv = *reinterpret_cast<const f32x4*>(crow + d0);
      bf16x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = (bf16)fmaf(mul, acc[m][4 * rg + i], cv[i] * (1.0f / kCubeTokens));
      *reinterpret_cast<bf16x4*>(orow + d0) = o;
    }
}

// dQ of one query cube from the dS tiles the dK/dV pass stored (one 64 x 64
// bf16 tile per list entry, as dS^T: rows = keys).  4 waves; wave w: key
// half kh = w & 1 of every selected key tile, query half qh = w >> 1:
//   dQ^T += K^T dS^T               (m = d, n = queries, k = 32 keys)
// with K^T and dS^T both read transposed from their natural tiles, which
// stream in together (global->LDS, double buffered).  As in the dK/dV
// pass's products, dS enters as its bf16 rounding r; the exact dS rows sum
// to zero over each query's keys, so dQ = sum_j r_j K_j - (sum_j r_j) c0,
// with c0 the mean of the first listed key cube and the sum of the rounded
// values taken in fp32, removes the rounding residue along the keys'
// shared component and leaves errors of the size of r - dS times K - c0.
template <int D>
__global__ __launch_bounds__(256, 2) void fine_bwd_dq_ds_kernel(
    const bf16* __restrict__ kp, const bf16* __restrict__ ds,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ ids, int topk, int64_t n_ids,
    const float* __restrict__ dqc, const float* __restrict__ kc_mean,
    int nh, int nc, int Hg, int Wg, float scale, int n_logical, bf16* __restrict__ dq) {
  constexpr int MD = D / 32, TILE_CH = 64 * D / 8, DS_CH = 64 * 64 / 8;
  __shared__ __align__(256) u32x4 k_lds0[TILE_CH];
  __shared__ __align__(256) u32x4 k_lds1[TILE_CH];
  __shared__ __align__(256) u32x4 s_lds0[DS_CH];
  __shared__ __align__(256) u32x4 s_lds1[DS_CH];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ql = lane & 31, hf = lane >> 5;
  const int kh = wave & 1, qh = wave >> 1;
  // XCD-contiguous logical numbering as in the forward fine kernel
  const int per = (n_logical + 7) >> 3;
  const int blk = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (blk >= n_logical) return;
  const int bh = blk / nc, c = blk - bh * nc;
  const int64_t N = (int64_t)nc * 64;
  const int64_t bh_tiles = (int64_t)bh * nc;
  int64_t start;
  int n;
  list_range(offs, blk, topk, n_ids, &start, &n);
  const int32_t* list = ids + start;
  const int slot = 32 * qh + ql;

  f32x16 acc[MD];
#pragma unroll
  for (int m = 0; m < MD; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[m][r] = 0.f;
  float ssum = 0.f;  // this lane's share of sum_j r_j

  // Entry `e` of the lists (key cube kc): its K tile and its dS tile.  An
  // id outside [0, nc) reads cube 0 and is skipped.
  auto copy_tile = [&](int64_t e, int kc, int buf) {
    kc = cube_or_0(kc, nc);
    dma_tile<D>(kp + (bh_tiles + kc) * 64 * D, buf ? k_lds1 : k_lds0, wave, lane);
    dma_tile<64>(ds + e * 4096, buf ? s_lds1 : s_lds0, wave, lane);
  };
  if (n > 0) copy_tile(start, list[0], 0);
  // transposed reads of rows (keys) 32kh .. 32kh + 31: of the K tile, column
  // blocks 0 .. MD-1; of the dS^T tile, column block qh (queries 32qh ..)
  const uint32_t tr_lo = tr_offset<D>(lane, 0) + 32 * kh * D * 2;
  const uint32_t tr_hi = tr_offset<D>(lane, 1) + 32 * kh * D * 2;
  const uint32_t sr_lo = tr_offset<64>(lane, 0) + 32 * kh * 64 * 2;
  const uint32_t sr_hi = tr_offset<64>(lane, 1) + 32 * kh * 64 * 2;

  for (int it = 0; it < n; ++it) {
    const int buf = it & 1;
    const bool tile_ok = cube_ok(list[it], nc);
    wait_vmcnt<0>();
    __syncthreads();
    if (it + 1 < n) copy_tile(start + it + 1, list[it + 1], buf ^ 1);
    if (!tile_ok) continue;
    const uint32_t kbase = lds_addr(buf ? k_lds1 : k_lds0);
    const uint32_t sbase = lds_addr(buf ? s_lds1 : s_lds0);
    bf16x8 ta[MD][2];
    tile_tr8_asm_cols<D, MD>(ta, kbase + tr_lo, kbase + tr_hi);
    bf16x8 dB[2];
    tile_tr8_asm<64, 2>(dB, (sbase + sr_lo) ^ ((uint32_t)qh << 6), (sbase + sr_hi) ^ ((uint32_t)qh << 6));
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) ssum += (float)dB[g][e];
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int m = 0; m < MD; ++m)
#pragma unroll
      for (int g = 0; g < 2; ++g)
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[m][g], dB[g], acc[m], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
  }

  ssum += swap_halves(ssum);  // over this wave's 32 keys of every tile
  // Sum the key halves: the kh = 1 wave hands its dQ^T and r sum to the
  // kh = 0 wave of the same query half through LDS.
  __syncthreads();  // all tile reads done; the buffers are free
  float* xo = reinterpret_cast<float*>(qh ? k_lds1 : k_lds0);  // 32 q x D floats
  float* xs = reinterpret_cast<float*>(qh ? s_lds1 : s_lds0);  // 32 q
  if (kh == 1) {
#pragma unroll
    for (int m = 0; m < MD; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[(m * 16 + r) * 64 + lane] = acc[m][r];
    if (hf == 0) xs[ql] = ssum;
  }
  __syncthreads();
  if (kh == 1) return;
  ssum += xs[ql];
  const float* c0 = kc_mean + (bh_tiles + (n > 0 ? cube_or_0(list[0], nc) : 0)) * D;

  const int b = bh / nh, h = bh - b * nh;
  const int tok = raster_tok(c, slot, Hg, Wg);
  const int64_t gidx = ((int64_t)b * N + tok) * nh + h;
  const float* qcr = dqc + (bh_tiles + c) * D;
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
        const float fine = (acc[m][r] + xo[(m * 16 + r) * 64 + lane]) - ssum * cc[i];
        o[i] = (bf16)fmaf(scale, fine, cq[i] * (1.0f / kCubeTokens));
      }
      *reinterpret_cast<bf16x4*>(dq + gidx * D + d0) = o;
    }
}

// dQ of one query cube: for each selected key cube, two halves of 32 keys.
//   phase A: thread (query i = t % 64, keys j = t / 64 + 4e, e < 8):
//            s = q_i.k_j, dP = dOf_i.v_j, P = exp(s s - lse_i),
//            dS = P (dP - Delta_i) into dsm[i][j]
//   phase B: thread (query i, dims d = t / 64 + 4m): dq_i[d] += sum_j dS k_j[d]
template <int D>
__global__ __launch_bounds__(256) void fine_bwd_dq_f32_kernel(
    const float* __restrict__ qp, const float* __restrict__ kp, const float* __restrict__ vp,
    const float* __restrict__ dofp, const float* __restrict__ lse_f, const float* __restrict__ delta,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ ids, int topk, int64_t n_ids,
    const float* __restrict__ dqc, int nh, int nc, int Hg, int Wg, float scale,
    float* __restrict__ dq) {
  constexpr int P1 = D + 1;
  __shared__ float qs[64 * P1], os[64 * P1];
  __shared__ float ks[32 * D], vs[32 * D];
  __shared__ float dsm[64 * 33];
  const int tid = threadIdx.x, i = tid & 63, w = tid >> 6;
  const int blk = blockIdx.x;
  const int bh = blk / nc, c = blk - bh * nc;
  const int64_t N = (int64_t)nc * 64;
  const int64_t bh_tiles = (int64_t)bh * nc;
  int64_t start;
  int n;
  list_range(offs, blk, topk, n_ids, &start, &n);
  copy_rows_f32<D>(qp + (bh_tiles + c) * 64 * D, qs, 64, P1);
  copy_rows_f32<D>(dofp + (bh_tiles + c) * 64 * D, os, 64, P1);
  const float lse = lse_f[(int64_t)bh * N + (int64_t)c * 64 + i];
  const float del = delta[(int64_t)bh * N + (int64_t)c * 64 + i];
  float acc[D / 4];
#pragma unroll
  for (int m = 0; m < D / 4; ++m) acc[m] = 0.f;
  for (int it = 0; it < n; ++it) {
    const int kc = ids[start + it];
    if (!cube_ok(kc, nc)) continue;  // not a key cube: no contribution
    for (int half = 0; half < 2; ++half) {
      __syncthreads();  // previous phase B done with ks, dsm
      const int64_t row0 = (bh_tiles + kc) * 64 + 32 * half;
      copy_rows_f32<D>(kp + row0 * D, ks, 32, D);
      copy_rows_f32<D>(vp + row0 * D, vs, 32, D);
      __syncthreads();
      float sv[8], dp[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) { sv[e] = 0.f; dp[e] = 0.f; }
#pragma unroll 8
      for (int d = 0; d < D; ++d) {
        const float qd = qs[i * P1 + d], od = os[i * P1 + d];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = w + 4 * e;
          sv[e] = fmaf(qd, ks[j * D + d], sv[e]);
          dp[e] = fmaf(od, vs[j * D + d], dp[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = expf(sv[e] * scale - lse);
        dsm[i * 33 + w + 4 * e] = p * (dp[e] - del);
      }
      __syncthreads();
#pragma unroll 4
      for (int j = 0; j < 32; ++j) {
        const float dsv = dsm[i * 33 + j];
#pragma unroll
        for (int m = 0; m < D / 4; ++m) acc[m] = fmaf(dsv, ks[j * D + w + 4 * m], acc[m]);
      }
    }
  }
  const int b = bh / nh, h = bh - b * nh;
  const int64_t gidx = ((int64_t)b * N + raster_tok(c, i, Hg, Wg)) * nh + h;
  const float* qcr = dqc + (bh_tiles + c) * D;
#pragma unroll
  for (int m = 0; m < D / 4; ++m) {
    const int d = w + 4 * m;
    dq[gidx * D + d] = fmaf(scale, acc[m], qcr[d] * (1.0f / kCubeTokens));
  }
}

// dK, dV of one key cube: for each query cube that selected it (ascending),
// two halves of 32 queries.
//   phase A: thread (key j = t % 64, queries i = t / 64 + 4e, e < 8):
//            P = exp(s q_i.k_j - lse_i), dS = P (dOf_i.v_j - Delta_i)
//   phase B: thread (key j, dims d = t / 64 + 4m):
//            dk_j[d] += sum_i dS q_i[d],  dv_j[d] += sum_i P dOf_i[d]
template <int D>
__global__ __launch_bounds__(256) void fine_bwd_dkdv_f32_kernel(
    const float* __restrict__ qp, const float* __restrict__ kp, const float* __restrict__ vp,
    const float* __restrict__ dofp, const float* __restrict__ lse_f, const float* __restrict__ delta,
    const int32_t* __restrict__ tr_offs, const int32_t* __restrict__ tr_ids, int64_t n_ids,
    const float* __restrict__ dkc, const float* __restrict__ dvc, int nh, int nc, int Hg, int Wg,
    float scale, float* __restrict__ dk, float* __restrict__ dv) {
  constexpr int P1 = D + 1;
  __shared__ float ks[64 * P1], vs[64 * P1];
  __shared__ float qs[32 * D], os[32 * D];
  __shared__ float pm[32 * 64], dsm[32 * 64];
  __shared__ float ls[32], ds_[32];
  const int tid = threadIdx.x, j = tid & 63, w = tid >> 6;
  const int blk = blockIdx.x;
  const int bh = blk / nc, kc = blk - bh * nc;
  const int64_t N = (int64_t)nc * 64;
  const int64_t bh_tiles = (int64_t)bh * nc;
  int64_t e0;
  int n;
  list_range(tr_offs, blk, 0, n_ids, &e0, &n);
  copy_rows_f32<D>(kp + (bh_tiles + kc) * 64 * D, ks, 64, P1);
  copy_rows_f32<D>(vp + (bh_tiles + kc) * 64 * D, vs, 64, P1);
  float ak[D / 4], av[D / 4];
#pragma unroll
  for (int m = 0; m < D / 4; ++m) { ak[m] = 0.f; av[m] = 0.f; }
  for (int it = 0; it < n; ++it) {
    const int c = cube_or_0(tr_ids[e0 + it], nc);  // the library's transposed lists always pass
    for (int half = 0; half < 2; ++half) {
      __syncthreads();  // previous phase B done with qs, os, pm, dsm
      const int64_t row0 = (bh_tiles + c) * 64 + 32 * half;
      copy_rows_f32<D>(qp + row0 * D, qs, 32, D);
      copy_rows_f32<D>(dofp + row0 * D, os, 32, D);
      if (tid < 32) ls[tid] = lse_f[(int64_t)bh * N + row0 - bh_tiles * 64 + tid];
      else if (tid < 64) ds_[tid - 32] = delta[(int64_t)bh * N + row0 - bh_tiles * 64 + tid - 32];
      __syncthreads();
      float sv[8], dp[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) { sv[e] = 0.f; dp[e] = 0.f; }
#pragma unroll 8
      for (int d = 0; d < D; ++d) {
        const float kd = ks[j * P1 + d], vd = vs[j * P1 + d];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = w + 4 * e;
          sv[e] = fmaf(qs[i * D + d], kd, sv[e]);
          dp[e] = fmaf(os[i * D + d], vd, dp[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = w + 4 * e;
        const float p = expf(sv[e] * scale - ls[i]);
        pm[i * 64 + j] = p;
        dsm[i * 64 + j] = p * (dp[e] - ds_[i]);
      }
      __syncthreads();
#pragma unroll 4
      for (int i = 0; i < 32; ++i) {
        const float pv = pm[i * 64 + j], dsv = dsm[i * 64 + j];
#pragma unroll
        for (int m = 0; m < D / 4; ++m) {
          const int d = w + 4 * m;
          ak[m] = fmaf(dsv, qs[i * D + d], ak[m]);
          av[m] = fmaf(pv, os[i * D + d], av[m]);
        }
      }
    }
  }
  const int b = bh / nh, h = bh - b * nh;
  const int64_t gidx = ((int64_t)b * N + raster_tok(kc, j, Hg, Wg)) * nh + h;
  const float* kcr = dkc + (bh_tiles + kc) * D;
  const float* vcr = dvc + (bh_tiles + kc) * D;
#pragma unroll
  for (int m = 0; m < D / 4; ++m) {
    const int d = w + 4 * m;
    dk[gidx * D + d] = fmaf(scale, ak[m], kcr[d] * (1.0f / kCubeTokens));
    dv[gidx * D + d] = av[m] + vcr[d] * (1.0f / kCubeTokens);
  }
}

// n_prod (1 or 2) batched products of one shape in one launch.
template <bool TA, bool TB>
hipError_t gemm(const GemmPair& g, int n_prod, int lda, int64_t sA, int ldb, int64_t sB, int ldc,
                int64_t sC, int M, int N, int K, int batch, hipStream_t st) {
  if (n_prod == 2 && 2 * batch > 65535) {  // past the grid's z limit: one launch per product
    const GemmPair second{{g.A[1], nullptr}, {g.B[1], nullptr}, {g.C[1], nullptr}, {g.alpha[1], 0.f}};
    const hipError_t e = gemm<TA, TB>(g, 1, lda, sA, ldb, sB, ldc, sC, M, N, K, batch, st);
    return e != hipSuccess ? e : gemm<TA, TB>(second, 1, lda, sA, ldb, sB, ldc, sC, M, N, K, batch, st);
  }
  dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64), (unsigned)(n_prod * batch));
  gemm_f32_kernel<TA, TB><<<grid, 256, 0, st>>>(g, batch, lda, sA, ldb, sB, ldc, sC, M, N, K);
  return hipGetLastError();
}

template <int D>
hipError_t launch_backward_d(const BackwardArgs& a, hipStream_t st) {
  const int nc = (a.T / 4) * (a.H / 4) * (a.W / 4);
  const int BH = a.B * a.heads;
  const float scale = 1.0f / sqrtf((float)D);
  hipError_t e;
#define VSA_TRY(x) do { e = (x); if (e != hipSuccess) return e; } while (0)
  if (a.bf16) {
    bwd_prep_kernel<D, bf16><<<(unsigned)(a.B * nc * a.heads), 256, 0, st>>>(
        (const bf16*)a.dout, (const bf16*)a.gc, (const bf16*)a.gf, a.of, a.oc, a.heads, a.T, a.H,
        a.W, (float*)a.dgc, (float*)a.dgf, a.delta, (bf16*)a.dofp, a.doc, a.deltac);
  } else {
    bwd_prep_kernel<D, float><<<(unsigned)(a.B * nc * a.heads), 256, 0, st>>>(
        (const float*)a.dout, (const float*)a.gc, (const float*)a.gf, a.of, a.oc, a.heads, a.T,
        a.H, a.W, (float*)a.dgc, (float*)a.dgf, a.delta, (float*)a.dofp, a.doc, a.deltac);
  }
  VSA_TRY(hipGetLastError());
  // coarse backward on the cube means
  const int64_t sq = (int64_t)nc * D, ss = (int64_t)nc * nc;
  // S = s Qc Kc^T and dP = dOc Vc^T in one launch
  VSA_TRY((gemm<false, true>(GemmPair{{a.qc, a.doc}, {a.kc, a.vc}, {a.S, a.dP}, {scale, 1.0f}}, 2,
                             D, sq, D, sq, nc, ss, nc, nc, D, BH, st)));
  const int64_t rows = (int64_t)BH * nc;
  coarse_softmax_grad_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, st>>>(a.S, a.dP, a.lse_c, a.deltac, nc, rows);
  VSA_TRY(hipGetLastError());
  // dQc = s dS Kc; then dKc = s dS^T Qc and dVc = P^T dOc in one launch
  VSA_TRY((gemm<false, false>(GemmPair{{a.dP, nullptr}, {a.kc, nullptr}, {a.dqc, nullptr}, {scale, 0.f}},
                              1, nc, ss, D, sq, D, sq, nc, D, nc, BH, st)));
  VSA_TRY((gemm<true, false>(GemmPair{{a.dP, a.S}, {a.qc, a.doc}, {a.dkc, a.dvc}, {scale, 1.0f}}, 2,
                             nc, ss, D, sq, D, sq, nc, D, nc, BH, st)));
  // transposed selection
  transpose_scatter_kernel<<<(unsigned)BH, 256, sizeof(int32_t) * (4 * nc + 4), st>>>(
      a.offs, a.ids, a.topk, a.n_ids, nc, a.tr_offs, a.tr_order, a.tr_tmp, a.bf16 ? a.tr_tmp_pos : nullptr);
  VSA_TRY(hipGetLastError());
  const int64_t n_lists = (int64_t)BH * nc;
  transpose_rank_kernel<<<(unsigned)((n_lists + 3) / 4), 256, 0, st>>>(
      a.tr_offs, a.tr_tmp, a.tr_tmp_pos, n_lists, a.n_ids, a.tr_ids, a.bf16 ? a.tr_pos : nullptr);
  VSA_TRY(hipGetLastError());
  const unsigned grid = (unsigned)(BH * nc);
  if (!a.bf16) {
    // the transposed lists are in natural key-cube order: tr_offs row = blk
    fine_bwd_dkdv_f32_kernel<D><<<grid, 256, 0, st>>>(
        (const float*)a.qp, (const float*)a.kp, (const float*)a.vp, (const float*)a.dofp,
        a.lse_f, a.delta, a.tr_offs, a.tr_ids, a.n_ids, a.dkc, a.dvc, a.heads, nc, a.H, a.W, scale,
        (float*)a.dk, (float*)a.dv);
    VSA_TRY(hipGetLastError());
    fine_bwd_dq_f32_kernel<D><<<grid, 256, 0, st>>>(
        (const float*)a.qp, (const float*)a.kp, (const float*)a.vp, (const float*)a.dofp,
        a.lse_f, a.delta, a.offs, a.ids, a.topk, a.n_ids, a.dqc, a.heads, nc, a.H, a.W, scale,
        (float*)a.dq);
    VSA_TRY(hipGetLastError());
    return hipSuccess;
  }
  fine_bwd_dkdv_kernel<D><<<((grid + 7u) / 8u) * 8u, 256, 0, st>>>(
      (const bf16*)a.qp, (const bf16*)a.kp, (const bf16*)a.vp, (const bf16*)a.dofp,
      a.lse_f, a.delta, a.tr_offs, a.tr_order, a.tr_ids, a.tr_pos, a.n_ids, a.dkc, a.dvc, a.heads, nc,
      a.H, a.W, scale, (int)grid, (bf16*)a.dk, (bf16*)a.dv, (bf16*)a.ds);
  VSA_TRY(hipGetLastError());
  fine_bwd_dq_ds_kernel<D><<<((grid + 7u) / 8u) * 8u, 256, 0, st>>>(
      (const bf16*)a.kp, (const bf16*)a.ds, a.offs, a.ids, a.topk, a.n_ids, a.dqc, a.kc, a.heads, nc,
      a.H, a.W, scale, (int)grid, (bf16*)a.dq);
  VSA_TRY(hipGetLastError());
#undef VSA_TRY
  return hipSuccess;
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, hipStream_t st) {
  return a.D == 128 ? launch_backward_d<128>(a, st) : launch_backward_d<64>(a, st);
}

}  // namespace vsa
