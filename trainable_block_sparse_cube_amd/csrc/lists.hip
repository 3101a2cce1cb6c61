// Padded per-row key-cube lists -> CSR (offsets + packed ids), the layout
// the variable-length fine stage reads ([VSA2-abs], "Improving Video Sparse
// Attention with Fine-grained Router and Sparse Rebasing", Abstract: each
// query may attend a variable number of key-value pairs).
//
//   scan_counts: one workgroup; offsets[r] = sum of counts[0..r), written
//                for r = 0..n (offsets[n] = total), 4 counts per thread per
//                pass with a running carry between passes
//   pack_lists:  one wave per row copies its count ids to offsets[row]
#include "vsa_device.h"
#include "vsa_launch.h"

namespace vsa {

namespace {

constexpr int kScanThreads = 1024;
constexpr int kScanPer = 4;

__global__ __launch_bounds__(kScanThreads) void scan_counts_kernel(const int32_t* __restrict__ counts,
                                                                   int n, int32_t* __restrict__ offsets) {
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
      v[e] = i0 + e < n ? counts[i0 + e] : 0;
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
  const int c = counts[row];
  const int64_t o = offsets[row];
  const int32_t* src = padded + (int64_t)row * k_max;
  for (int i = lane; i < c; i += 64) ids[o + i] = src[i];
}

}  // namespace

hipError_t launch_pack_lists(const int32_t* counts, const int32_t* padded, int n_rows, int k_max,
                             int32_t* offsets, int32_t* ids, hipStream_t st) {
  scan_counts_kernel<<<1, kScanThreads, 0, st>>>(counts, n_rows, offsets);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (n_rows == 0) return hipSuccess;
  pack_lists_kernel<<<(unsigned)((n_rows + 3) / 4), 256, 0, st>>>(counts, padded, n_rows, k_max,
                                                                  offsets, ids);
  return hipGetLastError();
}

}  // namespace vsa
