// Fine stage: block-sparse token attention over the selected cubes, with the
// gated combine fused into the epilogue.
//
// [VSA-abs] ("VSA: Faster Video Diffusion with Trainable Sparse Attention",
// Abstract): the fine stage computes token-level attention only inside the
// tiles picked by the coarse stage, in a block layout.  [VSA-sum, Approach]:
// each cube maps to one GPU tile and the two stages are combined through
// gates.  [VSA2-abs]: each query may attend a variable number of key-value
// pairs, so the key lists may be variable-length (CSR).
//
// bf16 kernel (MFMA, gfx950).  One workgroup = 4 waves = one query cube of
// 64 tokens.  Wave w takes query half qh = w & 1 (slots 32qh..+32) and key
// half kh = w >> 1 of every selected tile (keys 32kh..+32).  Per tile:
//   S^T (32 keys x 32 queries) = K * Q^T          D/16 x mfma 32x32x16 bf16
//   fp32 online softmax along keys: each lane holds one query column, so
//   the running max/sum are lane-local up to one exchange between the two
//   half-waves (v_permlane32_swap)
//   O^T (D x 32) += V^T * P^T                      D/16 x mfma 32x32x16
// Each wave keeps its own softmax state over its key half; the two halves
// are merged once at the end (split softmax).  K and V tiles (16 KB each
// at D = 128, both in natural [key][D] order) are copied straight from
// global memory into LDS (global_load_lds, no register staging) with an XOR
// chunk swizzle, double buffered: tile t+1 streams in while tile t is
// computed, one barrier per tile.  V^T operands come from transposing LDS
// reads (ds_read_b64_tr_b16).  The epilogue divides by the row sum, mixes
// in the coarse output with the two gates, rounds once to bf16 and
// scatters rows back to raster token order.  Query cubes run in the order
// given (the forward sorts them by where their lists' quarter and
// three-quarter entries lie, so that cubes sweeping similar key ranges
// share an XCD's L2 at the same time), or in natural order.
//
// fp32 kernel: plain VALU, one 256-thread workgroup per query cube; it
// serves the fp32 path, where no reduced precision is allowed.
#include "vsa_device.h"
#include "vsa_launch.h"

namespace vsa {

namespace {

__device__ __forceinline__ int raster_token(int c, int s, int Hg, int Wg) {
  const int W4 = Wg >> 2, H4 = Hg >> 2;
  const int ct = c / (H4 * W4), cy = (c / W4) % H4, cx = c % W4;
  return ((4 * ct + (s >> 4)) * Hg + 4 * cy + ((s >> 2) & 3)) * Wg + 4 * cx + (s & 3);
}

template <int D>
__global__ __launch_bounds__(256, 2) void fine_fwd_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kp, const bf16* __restrict__ vp,
    const float* __restrict__ oc, const bf16* __restrict__ gc, const bf16* __restrict__ gf,
    int nh, int nc, int Hg, int Wg,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ ids, int topk, int64_t n_ids,
    float scale_log2, int n_logical, const int32_t* __restrict__ order,
    bf16* __restrict__ out, float* __restrict__ lse_f, float* __restrict__ o_fine) {
  constexpr int KS = D / 16;          // k-steps of S^T over head_dim
  constexpr int TILE_CH = 64 * D / 8; // 16-byte chunks per K (and per V) tile
  constexpr int MD = D / 32;          // m-blocks of O^T
  // Lazy rescaling: the running max moves only when a tile's max exceeds
  // it by more than this many powers of two (exact; bounds p by 2^8).
  constexpr float kRescale = 8.f;

  // Two buffers (tile parity) of K and V.  Separate arrays, picked at run
  // time, so that the compiler adds no waits of its own for the copies; the
  // waits below (vmcnt + barrier) order every copy before its reads.
  __shared__ __align__(16) u32x4 k_lds0[TILE_CH];
  __shared__ __align__(16) u32x4 k_lds1[TILE_CH];
  __shared__ __align__(16) u32x4 v_lds0[TILE_CH];
  __shared__ __align__(16) u32x4 v_lds1[TILE_CH];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int qh = wave & 1;   // query half: slots 32*qh .. +32
  const int kh = wave >> 1;  // key half of every tile: keys 32*kh .. +32
  const int ql = lane & 31, hf = lane >> 5;

  // Logical block i: query cube (b*nh + h)*nc + c = order[i], or i itself
  // without an order.  Hardware block i runs on XCD i % 8 (round-robin
  // dispatch), so XCD x is given the contiguous logical range [x per,
  // (x + 1) per): the workgroups that share one XCD's L2 work on
  // neighbouring entries of the order, all of one or two heads: query
  // cubes with similar key lists (the sorted order), or neighbouring query
  // cubes (natural order), which select overlapping key cubes when the
  // inputs have spatial structure.  The grid is padded to a multiple of 8;
  // padding blocks exit at once.
  const int per = (n_logical + 7) >> 3;
  const int lblk = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (lblk >= n_logical) return;
  const int blk = order ? order[lblk] : lblk;
  if ((unsigned)blk >= (unsigned)n_logical) return;  // an order entry out of range runs nothing
  const int bh = blk / nc;
  const int c = blk - bh * nc;
  const int64_t N = (int64_t)nc * 64;
  int64_t start;
  int n;
  list_range(offs, blk, topk, n_ids, &start, &n);
  const int32_t* list = ids + start;
  const int64_t bh_tiles = (int64_t)bh * nc;
  const int b = bh / nh, h = bh - b * nh;

  // Copy the K and V tiles of key cube kc into buffer `buf`.  Both come
  // from contiguous cube-major tiles (each is re-read by about K query
  // cubes, and one contiguous 16 KB block streams better than 64 scattered
  // token rows).  An entry outside [0, nc) reads cube 0 and is skipped.
  auto copy_tile = [&](int kc, int buf) {
    kc = cube_or_0(kc, nc);
    dma_tile<D>(kp + (bh_tiles + kc) * 64 * D, buf ? k_lds1 : k_lds0, wave, lane);
    dma_tile<D>(vp + (bh_tiles + kc) * 64 * D, buf ? v_lds1 : v_lds0, wave, lane);
  };

  // Q^T operands, read once in place from the raster q: lane (query ql of
  // this half, half-wave hf) holds d = (D/2)*hf + 8s .. +8.
  bf16x8 qB[KS];
  {
    const int qtok = raster_token(c, 32 * qh + ql, Hg, Wg);
    const bf16* qrow = q + (((int64_t)b * N + qtok) * nh + h) * D + (D / 2) * hf;
#pragma unroll
    for (int s = 0; s < KS; ++s) qB[s] = *reinterpret_cast<const bf16x8*>(qrow + 8 * s);
  }
  if (n > 0) copy_tile(list[0], 0);

  f32x16 oacc[MD];
#pragma unroll
  for (int m = 0; m < MD; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[m][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int krow = 32 * kh + ql;  // this lane's K row (A operand of S^T)

  for (int it = 0; it < n; ++it) {
    const int buf = it & 1;
    const bool tile_ok = cube_ok(list[it], nc);
    wait_vmcnt<0>();   // this wave's copies of tile `it` have landed
    __syncthreads();   // all copies of tile `it` visible; buffer buf^1 free
    const u32x4* kb = buf ? k_lds1 : k_lds0;
    const u32x4* vb = buf ? v_lds1 : v_lds0;

    // Operands of both products are read from LDS up front, so the LDS
    // latency overlaps the MFMA chain instead of stalling each step.
    bf16x8 ka[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) ka[s] = tile_row8<D>(kb, krow, KS * hf + s);
    // V^T operands, read transposed from the natural V tile: keys
    // 32kh + 16g .. +16 in the order of pB.
    bf16x8 va[MD][2];
#pragma unroll
    for (int m = 0; m < MD; ++m)
#pragma unroll
      for (int g = 0; g < 2; ++g) va[m][g] = tile_tr8<D>(vb, 32 * kh + 16 * g, 32 * m, lane);
    __builtin_amdgcn_sched_barrier(0);  // keep the reads batched ahead of their MFMAs
    // The next tile's copy is queued only now: the compiler makes each
    // transposing read wait for every global->LDS copy in flight, so the
    // copy must not be in flight while they issue.  It still overlaps all
    // of this tile's arithmetic.
    if (it + 1 < n) copy_tile(list[it + 1], buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    if (!tile_ok) continue;

    // S^T (32 keys x 32 queries) = K[32kh..] * Q[32qh..]^T
    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s], qB[s], sacc, 0, 0, 0);

    // Online softmax over this wave's 32 keys, per query column ql.
    float mx = sacc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    mx = fmaxf(mx, swap_halves(mx)) * scale_log2;
    const bool grow = mx > m_run + kRescale;
    if (__any(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int m = 0; m < MD; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[m][r] *= alpha;
    }
    bf16x8 pB[2];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[8 * g + e], scale_log2, -m_run));
        l_run += p;
        pB[g][e] = (bf16)p;
      }

    // O^T += V^T[:, 32kh..] * P^T : two k-steps of 16 keys.
#pragma unroll
    for (int m = 0; m < MD; ++m)
#pragma unroll
      for (int g = 0; g < 2; ++g)
        oacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[m][g], pB[g], oacc[m], 0, 0, 0);
  }

  // Merge the two key halves (split softmax): waves with kh = 1 hand their
  // (m, l, O) to the kh = 0 wave of the same query half through LDS.
  l_run += swap_halves(l_run);
  __syncthreads();  // all tile reads done; the buffers are free
  float* xo = reinterpret_cast<float*>(qh ? k_lds1 : k_lds0);  // 32 q x D floats
  float* xs = reinterpret_cast<float*>(qh ? v_lds1 : v_lds0);  // m, l per query
  if (kh == 1) {
#pragma unroll
    for (int m = 0; m < MD; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[(m * 16 + r) * 64 + lane] = oacc[m][r];
    if (hf == 0) { xs[ql] = m_run; xs[32 + ql] = l_run; }
  }
  __syncthreads();
  if (kh == 1) return;
  const float m_o = xs[ql], l_o = xs[32 + ql];
  const float m_max = fmaxf(m_run, m_o);
  const float a_s = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_max);
  const float a_o = m_o == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_o - m_max);
  const float l_tot = l_run * a_s + l_o * a_o;
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;

  // Epilogue: normalise, gate-combine with the coarse output, scatter.
  const int slot = 32 * qh + ql;
  const int tok = raster_token(c, slot, Hg, Wg);
  const int64_t gidx = ((int64_t)b * N + tok) * nh + h;
  const float g_c = (float)gc[gidx], g_f = (float)gf[gidx];
  const float* ocrow = oc + (bh_tiles + c) * D;
  bf16* orow = out + gidx * D;
  float* ofrow = o_fine ? o_fine + ((int64_t)bh * N + (int64_t)c * 64 + slot) * D : nullptr;
#pragma unroll
  for (int m = 0; m < MD; ++m)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = 32 * m + 8 * rg + 4 * hf;
      const f32x4 ocv = *reinterpret_cast<const f32x4*>(ocrow + d0);
      f32x4 of;
      bf16x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * rg + i;
        of[i] = (oacc[m][r] * a_s + xo[(m * 16 + r) * 64 + lane] * a_o) * inv;
        o[i] = (bf16)fmaf(g_c, ocv[i], g_f * of[i]);
      }
      *reinterpret_cast<bf16x4*>(orow + d0) = o;
      if (ofrow) *reinterpret_cast<f32x4*>(ofrow + d0) = of;
    }
  if (lse_f && hf == 0)
    lse_f[(int64_t)bh * N + (int64_t)c * 64 + slot] =
        l_tot > 0.f ? (m_max + log2f(l_tot)) * kLn2 : -INFINITY;
}

// fp32: one workgroup of 256 threads per query cube, plain fp32 vector
// arithmetic.  The cube's 64 query rows sit in LDS (rows padded by one float
// so that lanes reading one column of different rows hit distinct banks);
// each selected key tile is taken in two halves of 32 keys:
//   phase A: thread (query i = t % 64, keys j = t / 64 + 4e, e < 8) forms
//            s_ij = scale * q_i.k_j into an LDS row block;
//   phase B: thread (query i, dims d = t / 64 + 4m) updates the running
//            max, rescales, and accumulates exp(s_ij - max) v_j[d].
// The four threads of a query row keep identical softmax statistics.
template <int D>
__global__ __launch_bounds__(256) void fine_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kp, const float* __restrict__ vp,
    const float* __restrict__ oc, const float* __restrict__ gc, const float* __restrict__ gf,
    int nh, int nc, int Hg, int Wg,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ ids, int topk, int64_t n_ids,
    float scale, float* __restrict__ out, float* __restrict__ lse_f, float* __restrict__ o_fine) {
  constexpr int P1 = D + 1;
  __shared__ float qs[64 * P1];
  __shared__ float ks[32 * D], vs[32 * D];
  __shared__ float sm[64 * 33];
  const int tid = threadIdx.x, i = tid & 63, w = tid >> 6;
  const int blk = blockIdx.x;
  const int bh = blk / nc;
  const int c = blk - bh * nc;
  const int64_t N = (int64_t)nc * 64;
  const int b = bh / nh, h = bh - b * nh;
  const int64_t bh_tiles = (int64_t)bh * nc;
  int64_t start;
  int n;
  list_range(offs, blk, topk, n_ids, &start, &n);

  // the cube's 64 query rows, gathered from raster order
  for (int e = tid; e < 64 * (D / 4); e += 256) {
    const int r = e / (D / 4), c4 = e - r * (D / 4);
    const int64_t tok = raster_token(c, r, Hg, Wg);
    const f32x4 x = *reinterpret_cast<const f32x4*>(q + (((int64_t)b * N + tok) * nh + h) * D + 4 * c4);
    float* d = qs + r * P1 + 4 * c4;
    d[0] = x[0]; d[1] = x[1]; d[2] = x[2]; d[3] = x[3];
  }
  float acc[D / 4];
#pragma unroll
  for (int m = 0; m < D / 4; ++m) acc[m] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  for (int it = 0; it < n; ++it) {
    const int kc = ids[start + it];
    if (!cube_ok(kc, nc)) continue;  // not a key cube: no contribution
    for (int half = 0; half < 2; ++half) {
      __syncthreads();  // previous phase B done with ks, vs, sm (and qs written)
      const int64_t row0 = (bh_tiles + kc) * 64 + 32 * half;
      copy_rows_f32<D>(kp + row0 * D, ks, 32, D);
      copy_rows_f32<D>(vp + row0 * D, vs, 32, D);
      __syncthreads();
      float sv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) {
        const float qd = qs[i * P1 + d];
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[e] = fmaf(qd, ks[(w + 4 * e) * D + d], sv[e]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sm[i * 33 + w + 4 * e] = sv[e] * scale;
      __syncthreads();
      float mx = m_run;
      for (int j = 0; j < 32; ++j) mx = fmaxf(mx, sm[i * 33 + j]);
      const float alpha = m_run == -INFINITY ? 0.f : expf(m_run - mx);
      m_run = mx;
      l_run *= alpha;
#pragma unroll
      for (int m = 0; m < D / 4; ++m) acc[m] *= alpha;
#pragma unroll 4
      for (int j = 0; j < 32; ++j) {
        const float p = expf(sm[i * 33 + j] - m_run);
        l_run += p;
#pragma unroll
        for (int m = 0; m < D / 4; ++m) acc[m] = fmaf(p, vs[j * D + w + 4 * m], acc[m]);
      }
    }
  }
  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
  const int tok = raster_token(c, i, Hg, Wg);
  const int64_t gidx = ((int64_t)b * N + tok) * nh + h;
  const float g_c = gc[gidx], g_f = gf[gidx];
  const float* ocrow = oc + (bh_tiles + c) * D;
  float* ofrow = o_fine ? o_fine + ((int64_t)bh * N + (int64_t)c * 64 + i) * D : nullptr;
#pragma unroll
  for (int m = 0; m < D / 4; ++m) {
    const int d = w + 4 * m;
    const float of = acc[m] * inv;
    out[gidx * D + d] = fmaf(g_c, ocrow[d], g_f * of);
    if (ofrow) ofrow[d] = of;
  }
  if (lse_f && w == 0)
    lse_f[(int64_t)bh * N + (int64_t)c * 64 + i] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
}

template <int D>
hipError_t launch_fine_d(const FineArgs& a, hipStream_t st) {
  const int nc = (a.T / 4) * (a.H / 4) * (a.W / 4);
  const unsigned grid = (unsigned)(a.B * a.heads * nc);
  const float scale = 1.0f / sqrtf((float)D);
  if (a.bf16) {
    fine_fwd_bf16_kernel<D><<<((grid + 7u) / 8u) * 8u, 256, 0, st>>>(
        (const bf16*)a.q, (const bf16*)a.kp, (const bf16*)a.vp, a.oc,
        (const bf16*)a.gc, (const bf16*)a.gf, a.heads, nc, a.H, a.W, a.offs, a.ids, a.topk,
        a.n_ids, scale * kLog2e, (int)grid, a.order, (bf16*)a.out, a.lse_f, a.o_fine);
  } else {
    fine_fwd_f32_kernel<D><<<grid, 256, 0, st>>>(
        (const float*)a.q, (const float*)a.kp, (const float*)a.vp, a.oc,
        (const float*)a.gc, (const float*)a.gf, a.heads, nc, a.H, a.W, a.offs, a.ids, a.topk,
        a.n_ids, scale, (float*)a.out, a.lse_f, a.o_fine);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fine_forward(const FineArgs& a, hipStream_t st) {
  return a.D == 128 ? launch_fine_d<128>(a, st) : launch_fine_d<64>(a, st);
}

}  // namespace vsa
