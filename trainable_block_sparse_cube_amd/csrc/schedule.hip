// Processing order of the fine stage's query cubes.
//
// Each query cube streams the tiles of its selected key cubes in list order
// (ascending for the coarse stage's own lists; [VSA-sum, Approach]: the
// fine stage attends inside the selected cubes, and the order within a
// list is free).  Query cubes whose lists cover similar key ranges sweep
// them at the same time, so when such cubes run side by side on one XCD
// more of their tile reads hit its L2.  This kernel sorts each (batch,
// head)'s query cubes by a Morton code of two points of their list: the
// entries at a quarter and at three quarters of it (indices n/4 and 3n/4),
// each scaled to 9 bits (id * 512 / Nc), interleaved with the first
// quarter's bits above the second's; cube index breaks ties.  Two points
// place a list by where its lower and upper halves lie, which groups lists
// more tightly than their middle entry alone (fewer tile reads beyond L2).
// One workgroup per (b, h) runs a stable least-significant-digit radix sort
// of the 18-bit codes in three passes of 6 bits, starting from cube order.
// In a pass every wave ranks its 64 entries among those with the same digit
// (peer masks from six ballots), the per-(digit, tile, wave) counts are
// scanned in (digit, tile, wave) order, and each entry moves to its digit's
// offset plus its rank, which keeps equal digits in input order.  The
// result only reorders work: every query cube's own arithmetic, hence the
// output, is unchanged.
#include "vsa_device.h"
#include "vsa_launch.h"

namespace vsa {

namespace {

constexpr int kOrderThreads = 1024;
constexpr int kOrderWaves = kOrderThreads / 64;
constexpr int kOrderMax = 4096;                        // cubes per (b, h) this sort holds
constexpr int kOrderTiles = kOrderMax / kOrderThreads;  // entries per thread
constexpr int kCoordBits = 9;                          // each list point scaled to 9 bits
constexpr int kKeyBits = 2 * kCoordBits;                // Morton code of the two points
constexpr int kDigitBits = 6;
constexpr int kPasses = (kKeyBits + kDigitBits - 1) / kDigitBits;  // 3
constexpr int kDigits = 1 << kDigitBits;
constexpr int kBins = kDigits * kOrderTiles * kOrderWaves;
static_assert(kPasses * kDigitBits >= kKeyBits, "passes cover the key");
static_assert(kBins % kOrderThreads == 0, "scan layout");

// Entry i of a list of n as a 9-bit coordinate (out-of-range ids count as 0).
__device__ __forceinline__ uint32_t list_point(const int32_t* __restrict__ ids, int64_t start, int i,
                                               int nc) {
  return (uint32_t)(((int64_t)cube_or_0(ids[start + i], nc) << kCoordBits) / nc);
}

// Bits of a above those of b, interleaved: bit j of a -> 2j + 1, of b -> 2j.
__device__ __forceinline__ uint32_t morton2(uint32_t a, uint32_t b) {
  uint32_t key = 0;
#pragma unroll
  for (int j = 0; j < kCoordBits; ++j) key |= (((a >> j) & 1u) << (2 * j + 1)) | (((b >> j) & 1u) << (2 * j));
  return key;
}

__global__ __launch_bounds__(kOrderThreads) void order_by_quartiles_kernel(
    const int32_t* __restrict__ offs, const int32_t* __restrict__ ids, int topk, int64_t n_ids,
    int nc, int32_t* __restrict__ order) {
  __shared__ uint32_t key_of[kOrderMax];  // sort key of each cube's list
  __shared__ uint16_t seq[2][kOrderMax];  // cubes in the current / next order
  __shared__ int32_t bins[kBins];         // counts per (digit, tile, wave), then their offsets
  __shared__ int32_t wsum[kOrderWaves];
  const int64_t base = (int64_t)blockIdx.x * nc;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int c = tid; c < nc; c += kOrderThreads) {
    int64_t start;
    int n;
    list_range(offs, base + c, topk, n_ids, &start, &n);
    // an empty list counts as key 0
    key_of[c] = n > 0 ? morton2(list_point(ids, start, n / 4, nc), list_point(ids, start, (3 * n) / 4, nc)) : 0u;
    seq[0][c] = (uint16_t)c;
  }
  const uint64_t below = (1ull << lane) - 1ull;
  for (int pass = 0; pass < kPasses; ++pass) {
    const uint16_t* src = seq[pass & 1];
    uint16_t* dst = seq[(pass & 1) ^ 1];
    for (int i = tid; i < kBins; i += kOrderThreads) bins[i] = 0;
    __syncthreads();
    int digit[kOrderTiles], rank[kOrderTiles];
#pragma unroll
    for (int u = 0; u < kOrderTiles; ++u) {
      const int idx = u * kOrderThreads + tid;
      const bool live = idx < nc;
      const int d = live ? (int)(key_of[src[idx]] >> (kDigitBits * pass)) & (kDigits - 1) : 0;
      uint64_t peers = __ballot(live);
#pragma unroll
      for (int b = 0; b < kDigitBits; ++b) {
        const uint64_t m = __ballot((d >> b) & 1);
        peers &= ((d >> b) & 1) ? m : ~m;
      }
      digit[u] = d;
      rank[u] = __popcll(peers & below);
      if (live && rank[u] == 0) bins[(d * kOrderTiles + u) * kOrderWaves + wave] = __popcll(peers);
    }
    __syncthreads();
    // exclusive scan of bins in (digit, tile, wave) order: thread t owns a run
    {
      constexpr int L = kBins / kOrderThreads;
      int v[L], s = 0;
#pragma unroll
      for (int i = 0; i < L; ++i) { v[i] = bins[tid * L + i]; s += v[i]; }
      int x = s;
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
      }
      if (lane == 63) wsum[wave] = x;
      __syncthreads();
      if (wave == 0) {
        int w = lane < kOrderWaves ? wsum[lane] : 0;
        for (int o = 1; o < kOrderWaves; o <<= 1) {
          const int y = __shfl_up(w, o);
          if (lane >= o) w += y;
        }
        if (lane < kOrderWaves) wsum[lane] = w;
      }
      __syncthreads();
      int prefix = x - s + (wave > 0 ? wsum[wave - 1] : 0);
#pragma unroll
      for (int i = 0; i < L; ++i) { bins[tid * L + i] = prefix; prefix += v[i]; }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kOrderTiles; ++u) {
      const int idx = u * kOrderThreads + tid;
      if (idx < nc) dst[bins[(digit[u] * kOrderTiles + u) * kOrderWaves + wave] + rank[u]] = src[idx];
    }
    __syncthreads();
  }
  for (int i = tid; i < nc; i += kOrderThreads) order[base + i] = (int32_t)(base + seq[kPasses & 1][i]);
}

}  // namespace

int order_max_cubes() { return kOrderMax; }

hipError_t launch_fine_order(const int32_t* offs, const int32_t* ids, int topk, int64_t n_ids,
                             int n_bh, int nc, int32_t* order, hipStream_t st) {
  order_by_quartiles_kernel<<<(unsigned)n_bh, kOrderThreads, 0, st>>>(offs, ids, topk, n_ids, nc, order);
  return hipGetLastError();
}

}  // namespace vsa
