// Processing order of the fine stage's query cubes.
//
// Each query cube streams the tiles of its selected key cubes in ascending
// cube order ([VSA-sum, Approach]: the fine stage attends inside the
// selected cubes; the order within a list is free).  Query cubes whose
// lists have similar middle entries sweep similar key ranges at the same
// time, so when such cubes run side by side on one XCD more of their tile
// reads hit its L2.  This kernel sorts each (batch, head)'s query cubes by
// the middle entry of their list (cube index breaking ties): one workgroup
// per (b, h), a bitonic sort of (middle id << 12 | cube) keys in LDS.  The
// result only reorders work: every query cube's own arithmetic, hence the
// output, is unchanged.
#include "vsa_device.h"
#include "vsa_launch.h"

namespace vsa {

namespace {

constexpr int kOrderThreads = 1024;
constexpr int kOrderMax = 4096;  // cubes per (b, h) this sort holds (>= the coarse stage's limit)

__global__ __launch_bounds__(kOrderThreads) void order_by_middle_kernel(
    const int32_t* __restrict__ offs, const int32_t* __restrict__ ids, int topk, int64_t n_ids,
    int nc, int P, int32_t* __restrict__ order) {
  __shared__ uint32_t key[kOrderMax];
  const int64_t base = (int64_t)blockIdx.x * nc;
  const int tid = threadIdx.x;
  for (int i = tid; i < P; i += kOrderThreads) {
    uint32_t kv = 0xFFFFFFFFu;  // padding sorts last
    if (i < nc) {
      int64_t start;
      int n;
      list_range(offs, base + i, topk, n_ids, &start, &n);
      const uint32_t mid = n > 0 ? (uint32_t)cube_or_0(ids[start + n / 2], nc) : 0u;
      kv = (mid << 12) | (uint32_t)i;
    }
    key[i] = kv;
  }
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += kOrderThreads) {
        const int l = i ^ j;
        if (l > i) {
          const uint32_t a = key[i], b = key[l];
          const bool ascending = (i & k) == 0;
          if ((a > b) == ascending) { key[i] = b; key[l] = a; }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < nc; i += kOrderThreads)
    order[base + i] = (int32_t)(base + (key[i] & 0xFFFu));
}

}  // namespace

int order_max_cubes() { return kOrderMax; }

hipError_t launch_fine_order(const int32_t* offs, const int32_t* ids, int topk, int64_t n_ids,
                             int n_bh, int nc, int32_t* order, hipStream_t st) {
  int P = 1;
  while (P < nc) P <<= 1;
  order_by_middle_kernel<<<(unsigned)n_bh, kOrderThreads, 0, st>>>(offs, ids, topk, n_ids, nc, P,
                                                                    order);
  return hipGetLastError();
}

}  // namespace vsa
