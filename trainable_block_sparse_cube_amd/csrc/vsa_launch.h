// Host-side launch interface between the C ABI (vsa_api.hip) and the
// kernel files.  Arguments are validated by the caller of these functions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vsa {

// Per tensor (q, k, v): raster source [B, N, heads, D]; optional outputs
// cube-major tiles [B, heads, Nc, 64, D] and fp32 means [B, heads, Nc, D].
struct PermutePoolPtrs {
  const void* src[3];
  void* nat[3];
  float* pooled[3];
  float* plain[3] = {nullptr, nullptr, nullptr};  // optional second copy of the means, plain layout
};
// Operand-ordered ("packed") pooled K and V for the coarse kernel's bf16
// path: each wave load of an MFMA operand block is one contiguous run.
// Per (b, h), keys are padded to packed_keys(nc) (a multiple of 32, zeros).
//   K: element (key j, dim d) at (j / 16) * 16 D + ((2 (d / 32) + (d % 8) / 4)
//      * 64 + 16 ((d % 32) / 8) + j % 16) * 4 + d % 4
//      (16-key blocks; lane 16 lg + li of k-step t, half hp, holds key li,
//      dims 32 t + 8 lg + 4 hp .. +4)
//   V: element (key j, dim d) at (j / 32) * 32 D + ((d / 16) * 64
//      + 16 ((j % 32) / 8) + d % 16) * 8 + j % 8
//      (32-key steps; lane 16 lg + li of column block cb holds column
//      16 cb + li, keys 8 lg .. +8 of the step)
__host__ __device__ inline int packed_keys(int nc) { return (nc + 31) & ~31; }
__host__ __device__ inline int64_t packed_k_index(int j, int d, int D) {
  return (int64_t)(j >> 4) * 16 * D +
         ((2 * (d >> 5) + ((d & 7) >> 2)) * 64 + 16 * ((d & 31) >> 3) + (j & 15)) * 4 + (d & 3);
}
__host__ __device__ inline int64_t packed_v_index(int j, int d, int D) {
  return (int64_t)(j >> 5) * 32 * D + (((d >> 4) * 64 + 16 * ((j & 31) >> 3) + (d & 15)) * 8) + (j & 7);
}

struct PermutePoolArgs {
  PermutePoolPtrs p;
  int B, heads, D, T, H, W;
  bool bf16;
  bool max_pool = false;   // per-channel max instead of the mean; no tiles written
  bool packed_kv = false;  // pooled K and V in the packed layouts (pitch packed_keys(nc))
  int n_tensors = 3;       // tensors 0 .. n_tensors - 1 of (q, k, v) are processed
};
hipError_t launch_permute_pool(const PermutePoolArgs& a, hipStream_t st);

struct CoarseArgs {
  const float *qc, *kc, *vc;
  int B, heads, D, nc, topk;
  float *oc, *lse;
  int32_t* sel;  // may be null when topk == 0
  bool x3;       // products as three bf16 MFMAs (bf16 inputs) instead of fp32 MFMA
  bool packed = false;  // (x3 only) kc, vc in the packed layouts, pitch packed_keys(nc)
  // Mass rule instead of top-K when counts is non-null: per row, the
  // shortest ranked prefix reaching `mass` of the coarse probability,
  // length clamped to [k_min, k_max], written to counts[row] and to sel at
  // stride k_max.
  float mass = 0.f;
  int k_min = 0, k_max = 0;
  int32_t* counts = nullptr;
};
// Padded lists -> CSR: offsets[0..n_rows] = exclusive scan of counts, ids
// packed in row order.
hipError_t launch_pack_lists(const int32_t* counts, const int32_t* padded, int n_rows, int k_max,
                             int32_t* offsets, int32_t* ids, hipStream_t st);
// Checks of caller-made key lists (CSR offsets, or fixed length `topk`
// when offs is null) against the fine kernels' preconditions.  Clears
// result[0..1], then counts into result[0] the offset faults (offs[0] != 0,
// a decrease, offs[n_rows] != n_ids) and into result[1] the lists holding
// an id outside [0, nc) or an id twice.  nc <= validate_max_cubes().
int validate_max_cubes();
hipError_t launch_validate_lists(const int32_t* offs, const int32_t* ids, int topk, int64_t n_ids,
                                 int n_rows, int nc, int32_t* result, hipStream_t st);
// Largest number of cubes the coarse kernel accepts.
int coarse_max_cubes(int D);
hipError_t launch_coarse_topk(const CoarseArgs& a, hipStream_t st);

struct FineArgs {
  const void* q;        // raster [B, N, heads, D]
  const void* kp;       // natural K tiles
  const void* vp;       // natural V tiles
  const float* oc;
  const void *gc, *gf;  // [B, N, heads]
  int B, heads, D, T, H, W;
  const int32_t* offs;  // null: fixed-length lists of `topk`
  const int32_t* ids;
  int topk;
  int64_t n_ids;        // entries in ids (CSR ranges are clamped to it)
  bool bf16;
  void* out;            // [B, N, heads, D]
  float* lse_f;         // [B, heads, N] cube-major, optional
  float* o_fine;        // [B, heads, N, D] cube-major, optional
  const int32_t* order = nullptr;  // processing order of the query cubes (global ids), optional
};
hipError_t launch_fine_forward(const FineArgs& a, hipStream_t st);
// Query cubes of each (b, h) sorted by a Morton code of the entries at a
// quarter and three quarters of their key list (cube index on ties), as
// global ids bh*nc + c, into order[n_bh*nc].
int order_max_cubes();
hipError_t launch_fine_order(const int32_t* offs, const int32_t* ids, int topk, int64_t n_ids,
                             int n_bh, int nc, int32_t* order, hipStream_t st);

// Backward (bf16 or fp32).  Inputs: raster dout, gates; cube-major tiles: qp
// from the backward's permute, kp, vp from the forward's saved state; fp32
// means (saved state); forward state (oc, lse_c,
// lse_f, of); key lists (offs null: fixed topk).  Scratch: delta [BH,N],
// dofp tiles, doc [BH,Nc,D], deltac [BH,Nc], S and dP [BH,Nc,Nc],
// dqc/dkc/dvc [BH,Nc,D], tr_offs [BH*Nc+1], tr_order [BH*Nc], tr_ids and
// tr_tmp (one int per list entry).
struct BackwardArgs {
  int B, heads, D, T, H, W;
  bool bf16;  // element type of inputs, tiles and dq/dk/dv: bf16 (MFMA) or fp32 (VALU)
  const void *dout, *gc, *gf;
  const void *qp, *kp, *vp;
  const float *qc, *kc, *vc;
  const float *oc, *lse_c, *lse_f, *of;
  const int32_t* offs;
  const int32_t* ids;
  int topk;
  int64_t n_ids;  // entries in ids, tr_ids, tr_tmp, tr_pos and tr_tmp_pos
  float* delta;
  void* dofp;
  float *doc, *deltac, *S, *dP, *dqc, *dkc, *dvc;
  int32_t *tr_offs, *tr_order, *tr_ids, *tr_tmp;
  int32_t *tr_pos, *tr_tmp_pos;  // per transposed entry: its index in ids (bf16 path)
  void* ds;                      // bf16 path: one 64 x 64 dS tile per entry of ids
  void *dq, *dk, *dv, *dgc, *dgf;
};
hipError_t launch_backward(const BackwardArgs& a, hipStream_t st);

}  // namespace vsa
