// Coarse stage: dense cube-to-cube attention on the pooled tensors and the
// top-K key cubes of every query cube.
//
// [VSA-sum, Approach] ("Faster Video Diffusion with Trainable Sparse
// Attention", summary page): the pooled cubes attend densely to each other,
// giving a coarse output per cube, and the coarse scores pick the top-K
// critical key cubes of each query cube.  [VSA-sum, Limitations]: this
// selection is a separate step, not fused into the fine attention kernel.
//
// One workgroup (8 waves) owns 16 query cubes of one (batch, head):
//   1. logits S[r][j] = scale * <qc_r, kc_j> for every key cube j with fp32
//      MFMA (operands straight from L2); the 16 x Nc block of logits stays
//      in LDS;
//   2. per row (one wave per row): top-K by (logit desc, index asc), ids
//      emitted ascending (candidate pruning + direct ranks, see select_row);
//      then the softmax statistics, and S is overwritten by the
//      probabilities;
//   3. Oc = P * vc with MFMA, vc operands read straight from L2.
// Two precisions of the products in steps 1 and 3, both accumulated in
// fp32:
//   * fp32 inputs: fp32 MFMA (v_mfma_f32_16x16x4f32), exact fp32 products;
//   * bf16 inputs: each fp32 operand x is split into bf16 hi = rn(x) and
//     lo = rn(x - hi), and a product x*y is taken as hi*hi + hi*lo + lo*hi
//     on bf16 MFMA (v_mfma_f32_16x16x32_bf16).  The dropped terms are below
//     about 3 * 2^-16 of |x*y|, so the logits keep about 16 significant
//     bits: index decisions differ from exact fp32 ones only where two
//     logits agree to about 1e-5 relative, far inside the 1e-3 near-tie
//     band of the selection rule, and the bf16 outputs are unaffected.  It
//     runs on the bf16 matrix rate instead of the fp32 one (16x).
// The softmax and the ranking are fp32 in both cases.  In the forward's
// bf16 path kc and vc arrive in packed operand order (one contiguous run per
// wave load); stage calls pass the plain [B, heads, Nc, D] means.
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

// x = hi + lo + r with hi = rn_bf16(x), lo = rn_bf16(x - hi) (x - hi is
// exact in fp32), |r| <= 2^-16 |x|.
__device__ __forceinline__ void split_bf16x8(const f32x4v a, const f32x4v b, bf16x8& hi,
                                             bf16x8& lo) {
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bf16 h = (bf16)x[e];
    hi[e] = h;
    lo[e] = (bf16)(x[e] - (float)h);
  }
}

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

constexpr int kNW = 8;        // waves per workgroup

// Row pitch of the logit block (floats): at least nc + 32 (a zero-padded
// last 32-key step) and a multiple of 8, so that both bf16 planes of a
// probability row start 16-byte aligned.
__host__ __device__ constexpr int coarse_pitch(int nc) { return (nc + 39) & ~7; }
constexpr int kCandCap = 256; // candidates ranked directly per row (at most)

// Candidate capacity per wave for nc cubes: 256 where two workgroups per CU
// still fit in LDS with it, else 128 where they fit with that (rows of up
// to 1120 cubes), else 256 (one workgroup per CU either way).  Rows with
// more candidates take the bitwise-search path, which gives the same ids.
// Rows of logits a workgroup holds in LDS: 16 while they fit with a full
// candidate scratch (up to 2272 cubes), else 8 (up to 3584 cubes).
int coarse_rows(int nc) {
  const size_t need16 = sizeof(float) * ((size_t)16 * coarse_pitch(nc) + (size_t)2 * kNW * kCandCap);
  return need16 <= kLdsBudget ? 16 : 8;
}

int coarse_cand_cap(int nc) {
  const size_t s_bytes = sizeof(float) * (size_t)coarse_rows(nc) * coarse_pitch(nc);
  const size_t half = kLdsBudget / 2;
  if (s_bytes + sizeof(float) * 2 * kNW * 256 <= half) return 256;
  if (s_bytes + sizeof(float) * 2 * kNW * 128 <= half) return 128;
  return kCandCap;
}

// Writes, ascending by index, every entry of the row with key > thr and
// the need_eq lowest-index entries with key == thr (at most `limit` ids).
// `keys` as in select_row; 0 marks entries past the end.
template <int MAXJ>
__device__ __forceinline__ void emit_by_threshold(const uint32_t (&keys)[MAXJ], int nc, uint32_t thr,
                                                  int need_eq, int limit, int lane,
                                                  int32_t* __restrict__ out) {
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  int base = 0, eq_seen = 0;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    if (64 * j < nc) {
      const int idx = 64 * j + lane;
      const bool valid = idx < nc && keys[j] != 0u;
      const bool gt = valid && keys[j] > thr;
      const bool eq = valid && keys[j] == thr;
      const uint64_t eq_mask = __ballot(eq);
      const bool take = gt || (eq && (eq_seen + __popcll(eq_mask & lt_mask)) < need_eq);
      const uint64_t take_mask = __ballot(take);
      const int pos = base + __popcll(take_mask & lt_mask);
      if (take && pos < limit) out[pos] = idx;
      base += __popcll(take_mask);
      eq_seen += __popcll(eq_mask);
    }
  }
}

// Top-K of one row held by one wave.  `keys` holds this lane's order keys
// of entries lane + 64 j (0 past the end; real order keys are never 0).
// Writes the topk entries with the largest (key, -index) to out[0..topk),
// ascending by index.  `ck`/`ci` are per-wave LDS scratch of `cap` words.
//
// For K <= 64 the K-th largest of the 64 per-lane maxima is a lower bound
// lo on the row's K-th largest key (the lane maxima are row entries), so
// only entries with key >= lo can be chosen, and every entry that beats
// such an entry is itself >= lo.  These candidates (typically a few dozen)
// are compacted in index order and each one's rank among them, counted
// directly, decides it: chosen iff fewer than K candidates beat it.  Larger
// K or candidate sets use a bitwise search for the K-th largest key.
template <int MAXJ>
__device__ __forceinline__ void select_row(const uint32_t (&keys)[MAXJ], int nc, int topk,
                                           int lane, uint32_t* __restrict__ ck,
                                           int32_t* __restrict__ ci, int32_t* __restrict__ out, int cap) {
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  uint32_t lo = 0;
  if (topk <= 64) {
    uint32_t lane_max = 0;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) lane_max = max(lane_max, keys[j]);
    lo = kth_largest_of_lanes(lane_max, topk);
  }
  int ncand = 0;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    if (64 * j < nc) {
      const bool in = keys[j] >= lo && keys[j] != 0u;
      const uint64_t m = __ballot(in);
      const int pos = ncand + __popcll(m & lt_mask);
      if (in && pos < cap) { ck[pos] = keys[j]; ci[pos] = 64 * j + lane; }
      ncand += __popcll(m);
    }
  }
  if (ncand <= cap) {
    __builtin_amdgcn_wave_barrier();
    int base = 0;
    for (int i0 = 0; i0 < ncand; i0 += 64) {
      const int i = i0 + lane;
      const uint32_t ki = i < ncand ? ck[i] : 0u;
      // Count the candidates that beat candidate i: 64 at a time held one
      // per lane, broadcast to the wave with readlane (no LDS round trip
      // per comparison).
      int beaten = 0;
      for (int c0 = 0; c0 < ncand; c0 += 64) {
        const uint32_t kl = c0 + lane < ncand ? ck[c0 + lane] : 0u;
        const int m = min(64, ncand - c0);
        for (int c = 0; c < m; ++c) {
          const uint32_t kc = __builtin_amdgcn_readlane(kl, c);
          beaten += (kc > ki) | ((kc == ki) & (c0 + c < i));
        }
      }
      const bool take = i < ncand && beaten < topk;
      const uint64_t tm = __ballot(take);
      const int pos = base + __popcll(tm & lt_mask);
      if (take && pos < topk) out[pos] = ci[i];
      base += __popcll(tm);
    }
    return;
  }
  // Fallback: K-th largest key by a greedy bitwise search over the row.
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = thr | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j)
      if (64 * j < nc) cnt += __popcll(__ballot(keys[j] >= c));
    if (cnt >= topk) thr = c;
  }
  int n_gt = 0;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j)
    if (64 * j < nc) n_gt += __popcll(__ballot(keys[j] > thr));
  emit_by_threshold<MAXJ>(keys, nc, thr, topk - n_gt, topk, lane, out);
}

// Length of a row's list under the mass rule: the shortest prefix of the
// ranking (order key descending, index ascending) whose probability mass
// reaches `mass` (unclamped; the caller clamps to [k_min, k_max]).  Also
// returns the threshold key thr and the count n_gt of entries above it, so
// an unclamped list is emitted directly: the entries above thr plus the
// first n - n_gt ties at thr.  e[j] * inv is the
// probability of entry 64 j + lane (0 past the end).  The mass of all
// entries with key >= t falls as t grows, so the largest t whose mass still
// reaches `mass` comes from a greedy bitwise search (wave sums are
// bitwise uniform across lanes); the entries strictly above it carry less
// than `mass`, and entries equal to it (bitwise-equal logits, hence equal
// probabilities) are added lowest id first until the mass is reached.
// Total mass below `mass` (rounding) gives every entry.
template <int MAXJ>
__device__ __forceinline__ int mass_length(const uint32_t (&keys)[MAXJ], const float (&e)[MAXJ],
                                           float inv, int nc, float mass, uint32_t& thr_out,
                                           int& n_gt_out) {
  float p[MAXJ];
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) p[j] = e[j] * inv;
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = thr | (1u << bit);
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j)
      if (64 * j < nc) a += keys[j] >= c ? p[j] : 0.f;
    if (wave_sum(a) >= mass) thr = c;
  }
  int n_gt = 0, n_eq = 0;
  float m_gt = 0.f, p_eq = 0.f;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    if (64 * j < nc) {
      const bool valid = keys[j] != 0u;
      const bool gt = valid && keys[j] > thr, eq = valid && keys[j] == thr;
      n_gt += __popcll(__ballot(gt));
      n_eq += __popcll(__ballot(eq));
      m_gt += gt ? p[j] : 0.f;
      p_eq = fmaxf(p_eq, eq ? p[j] : 0.f);
    }
  }
  m_gt = wave_sum(m_gt);
  p_eq = wave_max(p_eq);
  int n = n_gt;
  for (float acc = m_gt; n - n_gt < n_eq && acc < mass; ++n) acc += p_eq;
  thr_out = thr;
  n_gt_out = n_gt;
  return n;
}

// One workgroup: R = 16 query rows of one (batch, head), 8 waves.  With PK
// (the forward's bf16 path) the pooled K and V come in the packed operand
// order, so that every load of phases 1 and 3 is one contiguous run.
// Matrix products use v_mfma_f32_16x16x4f32 (fp32 in, fp32 accumulate).
// Lane l of a 16x16x4 step supplies row/column l % 16 and k-slice l / 16.
template <int D, int MAXJ, bool X3, bool PK>
__global__ __launch_bounds__(64 * kNW, 1) void coarse_topk_kernel(
    const float* __restrict__ qc, const float* __restrict__ kc,
    const float* __restrict__ vc, int nc, int topk, float scale,
    float* __restrict__ oc, float* __restrict__ lse, int32_t* __restrict__ sel,
    float mass, int k_min, int k_max, int32_t* __restrict__ counts, int cand_cap, int rows) {
  // The MFMA tiles span R = 16 query rows; the workgroup owns the first
  // `rows` of them (16, or 8 for rows too long for 16 in LDS).  Rows past
  // `rows` are computed in step 1 but neither stored nor used.
  constexpr int R = 16;
  constexpr int DQ = D / 4;          // head_dim slice per lane group
  constexpr int NCW = D / 16;        // waves that own a 16-column output block
  extern __shared__ float lds[];
  const int s_pitch = coarse_pitch(nc);  // room for a zero-padded last key block
  float* S = lds;                      // [R][s_pitch]
  uint32_t* cand_k = reinterpret_cast<uint32_t*>(S + rows * s_pitch);  // [kNW][cand_cap]
  int32_t* cand_i = reinterpret_cast<int32_t*>(cand_k + kNW * cand_cap);

  const int bh = blockIdx.y;
  const int row0 = blockIdx.x * rows;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, lg = lane >> 4;
  const float* qcb = qc + (int64_t)bh * nc * D;
  // PK: kc and vc in the packed (operand-ordered) layouts, keys padded
  static_assert(X3 || !PK, "packed layouts serve the bf16 x 3 path");
  const int64_t kv_pitch = PK ? packed_keys(nc) : nc;
  const float* kcb = kc + (int64_t)bh * kv_pitch * D;
  const float* vcb = vc + (int64_t)bh * kv_pitch * D;

  if constexpr (X3) {
    // ---- 1. logits, bf16 x 3.  k-step t (32 of head_dim): lane group lg
    // supplies d = 32t + 8lg .. +8 of its row (A: query row li, B: key li).
    // Wave w takes key blocks 16w, 16w + 16 kNW, ...; the next block's
    // operands are fetched while the current one is multiplied.
    constexpr int KT = D / 32;
    bf16x8 qh[KT], ql[KT];
    {
      const int row = min(row0 + li, nc - 1);  // rows past the end are never used
      const f32x4v* src = reinterpret_cast<const f32x4v*>(qcb + (int64_t)row * D + 8 * lg);
#pragma unroll
      for (int t = 0; t < KT; ++t) split_bf16x8(src[8 * t], src[8 * t + 1], qh[t], ql[t]);
    }
    auto load_k = [&](int j0, f32x4v (&kb)[2 * KT]) {
      if constexpr (PK) {  // one contiguous KB per load (block j0 / 16)
        const f32x4v* src = reinterpret_cast<const f32x4v*>(kcb + (int64_t)j0 * D) + lane;
#pragma unroll
        for (int i = 0; i < 2 * KT; ++i) kb[i] = src[64 * i];
      } else {
        const f32x4v* src =
            reinterpret_cast<const f32x4v*>(kcb + (int64_t)min(j0 + li, nc - 1) * D + 8 * lg);
#pragma unroll
        for (int t = 0; t < KT; ++t) { kb[2 * t] = src[8 * t]; kb[2 * t + 1] = src[8 * t + 1]; }
      }
    };
    f32x4v kb[2 * KT], kn[2 * KT];
    if (16 * wave < nc) load_k(16 * wave, kn);
    for (int j0 = 16 * wave; j0 < nc; j0 += 16 * kNW) {
#pragma unroll
      for (int i = 0; i < 2 * KT; ++i) kb[i] = kn[i];
      if (j0 + 16 * kNW < nc) load_k(j0 + 16 * kNW, kn);
      f32x4v acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        bf16x8 kh, kl;
        split_bf16x8(kb[2 * t], kb[2 * t + 1], kh, kl);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[t], kh, acc, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[t], kl, acc2, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql[t], kh, acc2, 0, 0, 0);
      }
      const int key = j0 + li;
      if (key < nc) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * lg + r < rows) S[(4 * lg + r) * s_pitch + key] = (acc[r] + acc2[r]) * scale;
      }
    }
  } else {
    // ---- 1. logits.  Contraction over head_dim: lane group lg covers
    // d in [lg*DQ, lg*DQ + DQ), one element per k-step.  Wave w takes key
    // blocks 16w, 16w + 16 kNW, ...; the next block's operands are fetched
    // while the current one is multiplied.
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
    for (int j0 = 16 * wave; j0 < nc; j0 += 16 * kNW) {
  #pragma unroll
      for (int i = 0; i < DQ / 4; ++i) kb[i] = kn[i];
      if (j0 + 16 * kNW < nc) load_k(j0 + 16 * kNW, kn);
      f32x4v acc = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
      for (int i = 0; i < DQ / 4; ++i)
  #pragma unroll
        for (int e = 0; e < 4; ++e)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[i][e], kb[i][e], acc, 0, 0, 0);
      const int key = j0 + li;
      if (key < nc) {
  #pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * lg + r < rows) S[(4 * lg + r) * s_pitch + key] = acc[r] * scale;
      }
    }
  }
  __syncthreads();

  // ---- 2. per-row top-K and softmax, one wave per row
  for (int rr = wave; rr < rows; rr += kNW) {
    const int row = row0 + rr;
    float* Srow = S + rr * s_pitch;
    if (row >= nc) {  // keep padded rows finite for phase 3
      for (int j = lane; j < s_pitch; j += 64) Srow[j] = 0.f;
      continue;
    }
    // The row stays in registers: entry 64 j + lane in sv[j].
    float sv[MAXJ];
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      const int idx = 64 * j + lane;
      sv[j] = (64 * j < nc && idx < nc) ? Srow[idx] : -INFINITY;
    }
    uint32_t keys[MAXJ];
    if (topk > 0 || counts) {
#pragma unroll
      for (int j = 0; j < MAXJ; ++j) keys[j] = sv[j] == -INFINITY ? 0u : order_key(sv[j]);
    }
    if (topk > 0 && !counts)
      select_row<MAXJ>(keys, nc, topk, lane, cand_k + wave * cand_cap, cand_i + wave * cand_cap,
                       sel + ((int64_t)bh * nc + row) * topk, cand_cap);
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) m = fmaxf(m, sv[j]);
    m = wave_max(m);
    // exp(x) as 2^(x log2 e): one v_exp_f32 per entry (2^-inf = 0 past the end).
    const float m2 = m * kLog2e;
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      sv[j] = __builtin_amdgcn_exp2f(fmaf(sv[j], kLog2e, -m2));
      z += sv[j];
    }
    z = wave_sum(z);
    const float inv = 1.0f / z;
    if (counts) {  // mass rule: this row's length, then its top-n by the same ranking
      uint32_t thr;
      int n_gt;
      const int n_raw = mass_length<MAXJ>(keys, sv, inv, nc, mass, thr, n_gt);
      const int n = min(max(n_raw, k_min), k_max);
      if (lane == 0) counts[(int64_t)bh * nc + row] = n;
      int32_t* out = sel + ((int64_t)bh * nc + row) * k_max;
      if (n == n_raw)  // the top n are the entries above thr and the first ties at thr
        emit_by_threshold<MAXJ>(keys, nc, thr, n - n_gt, n, lane, out);
      else
        select_row<MAXJ>(keys, nc, n, lane, cand_k + wave * cand_cap, cand_i + wave * cand_cap, out,
                         cand_cap);
    }
    if constexpr (X3) {
      // P as two bf16 planes in the row's own storage: hi at [0, s_pitch),
      // lo at [s_pitch, 2 s_pitch) (bf16 elements), zero past nc.
      bf16* ph = reinterpret_cast<bf16*>(Srow);
      bf16* pl = ph + s_pitch;
#pragma unroll
      for (int j = 0; j < MAXJ; ++j) {
        const int idx = 64 * j + lane;
        if (64 * j < nc && idx < nc) {
          const float pv = sv[j] * inv;
          const bf16 h = (bf16)pv;
          ph[idx] = h;
          pl[idx] = (bf16)(pv - (float)h);
        }
      }
      for (int j = nc + lane; j < s_pitch; j += 64) { ph[j] = (bf16)0.f; pl[j] = (bf16)0.f; }
    } else {
#pragma unroll
      for (int j = 0; j < MAXJ; ++j) {
        const int idx = 64 * j + lane;
        if (64 * j < nc && idx < nc) Srow[idx] = sv[j] * inv;
      }
      for (int j = nc + lane; j < s_pitch; j += 64) Srow[j] = 0.f;  // padded key block
    }
    if (lane == 0) lse[(int64_t)bh * nc + row] = m + logf(z);
  }
  __syncthreads();

  if constexpr (X3) {
    // ---- 3. Oc = P * vc, bf16 x 3.  Wave w owns output columns
    // [16 cb, 16 cb + 16), cb = w % (D/16), and every (kNW/(D/16))-th
    // 32-key step starting at w / (D/16).  k-step keys j0 + 8lg .. +8:
    // P from the row's bf16 planes (A: row li), vc read straight from L2
    // (B: column li) and split in registers; the next step prefetched.
    constexpr int NCB = D / 16;
    constexpr int NKS = kNW / NCB;
    const int cb = wave % NCB, kq = wave / NCB;
    const int col = 16 * cb + li;
    // rows past `rows` read the last held row: their outputs are dropped
    const bf16* prow = reinterpret_cast<const bf16*>(S + min(li, rows - 1) * s_pitch);
    auto load_v = [&](int j0, float (&vbuf)[8]) {
      if constexpr (PK) {  // this lane's 8 keys of column col, contiguous (step j0 / 32)
        const f32x4v* src = reinterpret_cast<const f32x4v*>(vcb + (int64_t)j0 * D + (cb * 64 + lane) * 8);
        const f32x4v a = src[0], b = src[1];
        vbuf[0] = a.x; vbuf[1] = a.y; vbuf[2] = a.z; vbuf[3] = a.w;
        vbuf[4] = b.x; vbuf[5] = b.y; vbuf[6] = b.z; vbuf[7] = b.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = min(j0 + 8 * lg + e, nc - 1);  // P is 0 past the end
          vbuf[e] = vcb[(int64_t)key * D + col];
        }
      }
    };
    f32x4v oacc = {0.f, 0.f, 0.f, 0.f}, oacc2 = {0.f, 0.f, 0.f, 0.f};
    float vb[8], vn[8];
    if (32 * kq < nc) load_v(32 * kq, vn);
    for (int j0 = 32 * kq; j0 < nc; j0 += 32 * NKS) {
#pragma unroll
      for (int e = 0; e < 8; ++e) vb[e] = vn[e];
      if (j0 + 32 * NKS < nc) load_v(j0 + 32 * NKS, vn);
      bf16x8 vh, vl;
      split_bf16x8(f32x4v{vb[0], vb[1], vb[2], vb[3]}, f32x4v{vb[4], vb[5], vb[6], vb[7]}, vh, vl);
      const bf16x8 pa = *reinterpret_cast<const bf16x8*>(prow + j0 + 8 * lg);
      const bf16x8 pb = *reinterpret_cast<const bf16x8*>(prow + s_pitch + j0 + 8 * lg);
      oacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vh, oacc, 0, 0, 0);
      oacc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vl, oacc2, 0, 0, 0);
      oacc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb, vh, oacc2, 0, 0, 0);
    }
    oacc += oacc2;
    if constexpr (NKS > 1) {
      // key splits of one column block summed through the (now free)
      // candidate scratch
      static_assert(NKS == 2, "two key splits at head_dim 64");
      float* red = reinterpret_cast<float*>(cand_k);
      if (kq == 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(cb * 4 + r) * 64 + lane] = oacc[r];
      }
      __syncthreads();
      if (kq == 1) return;
#pragma unroll
      for (int r = 0; r < 4; ++r) oacc[r] += red[(cb * 4 + r) * 64 + lane];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 4 * lg + r;
      if (row < nc && 4 * lg + r < rows) oc[((int64_t)bh * nc + row) * D + col] = oacc[r];
    }
  } else {
    // ---- 3. Oc = P * vc.  Wave w < D/16 owns output columns [16w, 16w + 16);
    // contraction over keys, lane group lg taking key j0 + 4t + lg at k-step
    // t.  B operands come straight from L2 (vc of one head is small), the
    // next 32-key block prefetched during the current.
    if (wave < NCW) {
      f32x4v oacc = {0.f, 0.f, 0.f, 0.f};
      const int col = 16 * wave + li;
      auto load_v = [&](int j0, float (&vbuf)[8]) {
  #pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int key = min(j0 + 4 * t + lg, nc - 1);  // P is 0 past the end
          vbuf[t] = vcb[(int64_t)key * D + col];
        }
      };
      float vb[8], vn[8];
      load_v(0, vn);
      for (int j0 = 0; j0 < nc; j0 += 32) {
  #pragma unroll
        for (int t = 0; t < 8; ++t) vb[t] = vn[t];
        if (j0 + 32 < nc) load_v(j0 + 32, vn);
  #pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float pa = S[min(li, rows - 1) * s_pitch + j0 + 4 * t + lg];
          oacc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa, vb[t], oacc, 0, 0, 0);
        }
      }
  #pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + 4 * lg + r;
        if (row < nc && 4 * lg + r < rows) oc[((int64_t)bh * nc + row) * D + col] = oacc[r];
      }
    }
  }
}

size_t coarse_lds_bytes(int nc) {
  const int s_pitch = coarse_pitch(nc);
  return sizeof(float) * ((size_t)coarse_rows(nc) * s_pitch + (size_t)2 * kNW * coarse_cand_cap(nc));
}

template <int D, int MAXJ, bool X3, bool PK>
hipError_t launch_coarse_dj(const CoarseArgs& a, hipStream_t st) {
  const size_t lds = coarse_lds_bytes(a.nc);
  auto kern = coarse_topk_kernel<D, MAXJ, X3, PK>;
  // Allow this much dynamic LDS (host-side call, made on every launch: the
  // setting belongs to the current device, and the call is cheap).
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int rows = coarse_rows(a.nc);
  dim3 grid((unsigned)((a.nc + rows - 1) / rows), (unsigned)(a.B * a.heads));
  kern<<<grid, 64 * kNW, lds, st>>>(a.qc, a.kc, a.vc, a.nc, a.topk, 1.0f / sqrtf((float)D),
                                a.oc, a.lse, a.sel, a.mass, a.k_min, a.k_max, a.counts,
                                coarse_cand_cap(a.nc), rows);
  return hipGetLastError();
}

template <int D, bool X3, bool PK>
hipError_t launch_coarse_d(const CoarseArgs& a, hipStream_t st) {
  if (a.nc <= 16 * 64) return launch_coarse_dj<D, 16, X3, PK>(a, st);
  if (a.nc <= 20 * 64) return launch_coarse_dj<D, 20, X3, PK>(a, st);
  if (a.nc <= 40 * 64) return launch_coarse_dj<D, 40, X3, PK>(a, st);
  return launch_coarse_dj<D, 56, X3, PK>(a, st);  // the most chunks that fit in registers
}

}  // namespace

int coarse_max_cubes(int D) {
  (void)D;
  // 8 rows of logits plus candidate scratch in LDS, and at most 56 key
  // chunks of 64 per row (the row a wave ranks sits in its registers).
  const int max_pitch = (int)((kLdsBudget / sizeof(float) - 2 * kNW * kCandCap) / 8) & ~7;
  const int by_lds = max_pitch - 32;  // largest nc with coarse_pitch(nc) <= max_pitch
  return by_lds < 56 * 64 ? by_lds : 56 * 64;
}

hipError_t launch_coarse_topk(const CoarseArgs& a, hipStream_t st) {
  if (a.x3 && a.packed)
    return a.D == 128 ? launch_coarse_d<128, true, true>(a, st) : launch_coarse_d<64, true, true>(a, st);
  if (a.x3) return a.D == 128 ? launch_coarse_d<128, true, false>(a, st) : launch_coarse_d<64, true, false>(a, st);
  return a.D == 128 ? launch_coarse_d<128, false, false>(a, st) : launch_coarse_d<64, false, false>(a, st);
}

}  // namespace vsa
