// Padded per-row key-cube lists -> CSR (offsets + packed ids), the layout
// the variable-length fine stage reads ([VSA2-abs], "Improving Video Sparse
// Attention with Fine-grained Router and Sparse Rebasing", Abstract: each
// query may attend a variable number of key-value pairs).
//
//   scan_counts: one workgroup; offsets[r] = sum of counts[0..r), written
//                for r = 0..n (offsets[n] = total), 4 counts per thread per
//                pass with a running carry between passes
//   pack_lists:  one wave per row copies its count ids to offsets[row]
//
// Counts outside [0, k_max] are clamped, so the packed ids never exceed the
// n_rows * k_max capacity and no padded row is read past its end.
//
// validate_lists checks caller-made lists (CSR or fixed length) against
// the preconditions the fine kernels assume: offsets start at 0, never
// decrease and end at the number of ids; every id lies in [0, Nc); no id
// appears twice in one list.  One wave per list, with an LDS bitmap of the
// Nc cubes for the repeat test.
#include "vsa_device.h"
#include "vsa_launch.h"

namespace vsa {

namespace {

constexpr int kScanThreads = 1024;
constexpr int kValidateMaxCubes = 4096;
constexpr int kScanPer = 4;

__global__ __launch_bounds__(kScanThreads) void scan_counts_kernel(const int32_t* __restrict__ counts,
                                                                   int n, int k_max,
                                                                   int32_t* __restrict__ offsets) {
  __shared__ int32_t part[kScanThreads];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < n; base += kScanThreads * kScanPer) {
    const int i0 = base + tid * kScanPer;
    int v[kScanPer];
    int local = 0;
#pragma unroll
    for (int e = 0; e < kScanPer; ++e) {
      v[e] = i0 + e < n ? min(max(counts[i0 + e], 0), k_max) : 0;
      local += v[e];
    }
    part[tid] = local;
    __syncthreads();
    // inclusive Hillis-Steele scan of the per-thread sums
    for (int o = 1; o < kScanThreads; o <<= 1) {
      const int add = tid >= o ? part[tid - o] : 0;
      __syncthreads();
      part[tid] += add;
      __syncthreads();
    }
    const int carry = carry_s;
    int run = carry + part[tid] - local;  // exclusive prefix of this thread's first count
#pragma unroll
    for (int e = 0; e < kScanPer; ++e) {
      if (i0 + e < n) offsets[i0 + e] = run;
      run += v[e];
    }
    __syncthreads();  // every thread has read carry_s and part[]
    if (tid == kScanThreads - 1) carry_s = carry + part[tid];
    __syncthreads();
  }
  if (tid == 0) offsets[n] = carry_s;
}

__global__ __launch_bounds__(256) void pack_lists_kernel(const int32_t* __restrict__ counts,
                                                         const int32_t* __restrict__ padded, int n,
                                                         int k_max, const int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ ids) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= n) return;
  const int c = min(max(counts[row], 0), k_max);
  const int64_t o = offsets[row];
  const int32_t* src = padded + (int64_t)row * k_max;
  for (int i = lane; i < c; i += 64) ids[o + i] = src[i];
}

constexpr int kValidateWords = kValidateMaxCubes / 32;

__global__ void validate_clear_kernel(int32_t* __restrict__ result) {
  if (threadIdx.x < 2) result[threadIdx.x] = 0;
}

__global__ __launch_bounds__(256) void validate_lists_kernel(
    const int32_t* __restrict__ offs, const int32_t* __restrict__ ids, int topk, int64_t n_ids,
    int n_rows, int nc, int32_t* __restrict__ result) {
  __shared__ uint32_t seen[4][kValidateWords];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= n_rows) return;  // whole waves only; no workgroup barrier below
  if (offs && lane == 0) {
    const int64_t a = offs[row], b = offs[row + 1];
    const bool bad = b < a || (row == 0 && a != 0) || (row == n_rows - 1 && b != n_ids);
    if (bad) atomicAdd(&result[0], 1);
  }
  uint32_t* bits = seen[wave];
  const int words = (nc + 31) >> 5;
  for (int w = lane; w < words; w += 64) bits[w] = 0;
  // the wave's clears land before its own bitmap updates
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  int64_t s;
  int n;
  list_range(offs, row, topk, n_ids, &s, &n);
  bool bad = false;
  for (int i = lane; i < n; i += 64) {
    const int id = ids[s + i];
    if (!cube_ok(id, nc)) {
      bad = true;
    } else {
      const uint32_t bit = 1u << (id & 31);
      if (atomicOr(&bits[id >> 5], bit) & bit) bad = true;
    }
  }
  if (__any(bad) && lane == 0) atomicAdd(&result[1], 1);
}

}  // namespace

int validate_max_cubes() { return kValidateMaxCubes; }

hipError_t launch_validate_lists(const int32_t* offs, const int32_t* ids, int topk, int64_t n_ids,
                                 int n_rows, int nc, int32_t* result, hipStream_t st) {
  validate_clear_kernel<<<1, 64, 0, st>>>(result);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_rows == 0) return e;
  validate_lists_kernel<<<(unsigned)((n_rows + 3) / 4), 256, 0, st>>>(offs, ids, topk, n_ids, n_rows,
                                                                      nc, result);
  return hipGetLastError();
}

hipError_t launch_pack_lists(const int32_t* counts, const int32_t* padded, int n_rows, int k_max,
                             int32_t* offsets, int32_t* ids, hipStream_t st) {
  scan_counts_kernel<<<1, kScanThreads, 0, st>>>(counts, n_rows, k_max, offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (n_rows == 0) return hipSuccess;
  pack_lists_kernel<<<(unsigned)((n_rows + 3) / 4), 256, 0, st>>>(counts, padded, n_rows, k_max,
                                                                  offsets, ids);
  return hipGetLastError();
}

}  // namespace vsa
