// Device-side helpers shared by the gfx950 kernels: element types, MFMA
// operand vectors, bf16 rounding, cross-lane exchanges and the swizzled
// LDS cube tiles (global->LDS copies, row and transposed operand reads).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vsa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kCubeTokens = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// fptrunc to bf16 rounds to nearest even on gfx950 (v_cvt_pk_bf16_f32).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Value held by lane (l ^ 32) of the same wave.
__device__ __forceinline__ float swap_halves(float x) {
  uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  // r[0]: lanes 32..63 hold lanes 0..31's value; r[1]: lanes 0..31 hold
  // lanes 32..63's value.
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// ------------------------------------------------------------ key lists
// Entry range of list `row`: a fixed-length list of `topk` ids (offs null)
// or CSR offsets, each clamped to the id array [0, n_ids) so that a
// malformed offset array can never send a read outside it.  The library
// only promises meaningful results for well-formed lists (non-decreasing
// offsets from 0 to n_ids, ids in [0, Nc), no repeats within a list); for
// anything else it promises only that every access stays in bounds.
__device__ __forceinline__ void list_range(const int32_t* offs, int64_t row, int topk, int64_t n_ids,
                                           int64_t* start, int* n) {
  if (!offs) { *start = row * topk; *n = topk; return; }
  const int64_t s = min(max((int64_t)offs[row], (int64_t)0), n_ids);
  const int64_t e = min(max((int64_t)offs[row + 1], s), n_ids);
  *start = s;
  *n = (int)(e - s);
}

// A list entry names a key cube only if it lies in [0, nc); kernels read
// cube 0 in place of any other value and drop its contribution.
__device__ __forceinline__ bool cube_ok(int id, int nc) { return (unsigned)id < (unsigned)nc; }
__device__ __forceinline__ int cube_or_0(int id, int nc) { return cube_ok(id, nc) ? id : 0; }

// ------------------------------------------------------------ fp32 tiles
// Copy `rows` rows of D floats from src (contiguous) into dst with row
// pitch `pitch` floats, by the 256 threads of the workgroup (the fp32
// kernels; a pitch of D + 1 puts a column's rows on distinct banks).
template <int D>
__device__ __forceinline__ void copy_rows_f32(const float* __restrict__ src, float* dst, int rows, int pitch) {
  constexpr int V = D / 4;  // float4 per row
  for (int i = threadIdx.x; i < rows * V; i += 256) {
    const int r = i / V, c4 = i - r * V;
    const f32x4 x = *reinterpret_cast<const f32x4*>(src + (int64_t)r * D + 4 * c4);
    float* d = dst + r * pitch + 4 * c4;
    d[0] = x[0]; d[1] = x[1]; d[2] = x[2]; d[3] = x[3];
  }
}

// ------------------------------------------------------------ LDS tiles
// A cube tile is 64 rows (tokens) x D bf16, row-major, moved as 16-byte
// chunks (KCH = D/8 per row).  In LDS, logical chunk c of row r sits at
// physical chunk c ^ swz_tile<D>(r).  The MFMA kernels read a tile two
// ways: 16-byte row reads (one row per lane; 16 lanes share a chunk column
// and cover 16 consecutive rows) and ds_read_b64_tr_b16 transposed reads
// (per 16 lanes: 4 consecutive rows x 2 chunks; per 32 lanes: 4 rows x 4
// chunks).  The swizzle is linear over GF(2) in the row bits; its images of
// row bits 0..3 are independent (row reads: distinct chunks over 16 rows,
// and over 8 rows modulo 8 chunks), and the images of bits 0 and 1 differ in
// chunk bits 1-2 and in bits 2-3 (transposed reads).  So both access kinds
// fall on distinct banks with 32 or 64 banks of 4 bytes.
template <int D>
__device__ __forceinline__ int swz_tile(int row) {
  const int b0 = row & 1, b1 = (row >> 1) & 1, b2 = (row >> 2) & 1, b3 = (row >> 3) & 1;
  if constexpr (D == 128) return (6 * b0) ^ (10 * b1) ^ (1 * b2) ^ (2 * b3);
  else return (2 * b0) ^ (4 * b1) ^ (1 * b2) ^ (2 * b3);
}

// vmcnt-only wait (expcnt and lgkmcnt left at their maxima), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS traffic issued by the waves themselves (ds_*):
// waits for this wave's LDS operations, then meets the other waves.  Unlike
// __syncthreads() (whose LDS release also covers global->LDS copies), it
// does not wait for copies still in flight, so a copy of the next tile keeps
// streaming across it.  Only for LDS data that no copy in flight targets.
// The asm statement is also a compiler barrier for memory accesses.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One 16-byte global -> LDS copy per lane (global_load_lds); lane l of the
// wave writes LDS bytes [16 l, 16 l + 16) past `lds_wave_base` (wave-uniform).
__device__ __forceinline__ void copy16_to_lds(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

// Queue the copy of the contiguous tile `src` (64 x D bf16) into the LDS
// tile `dst` (swizzled), spread over the 4 waves of a 256-thread workgroup.
// Completion: wait_vmcnt in each wave, then a barrier.
template <int D>
__device__ __forceinline__ void dma_tile(const bf16* src, u32x4* dst, int wave, int lane) {
  constexpr int KCH = D / 8;
  constexpr int LD = 64 * KCH / 256;  // copies per wave
#pragma unroll
  for (int j = 0; j < LD; ++j) {
    const int P = (4 * j + wave) * 64 + lane;  // destination chunk
    const int row = P / KCH, phys = P % KCH;
    copy16_to_lds(src + (row * KCH + (phys ^ swz_tile<D>(row))) * 8, dst + (4 * j + wave) * 64);
  }
}

// 16-byte row read: logical chunk `chunk` of row `row` of an LDS tile.
template <int D>
__device__ __forceinline__ bf16x8 tile_row8(const u32x4* t, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(&t[row * (D / 8) + (chunk ^ swz_tile<D>(row))]);
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// A operand of one v_mfma_f32_32x32x16_bf16 step that contracts over tile
// rows: lane l gets column c0 + l%32 of rows
//   r0 + 4h + {0,1,2,3} and r0 + 8 + 4h + {0,1,2,3},   h = l / 32,
// i.e. the k-order in which a 32x32 accumulator holds rows r0 .. r0+15
// (register 8g + e of a block sits at row 16g + 8(e/4) + 4h + e%4), so a
// converted accumulator block can serve directly as the other operand.
// Built from two ds_read_b64_tr_b16: within 16 lanes, lane i receives
// element i % 4 of the 8-byte loads of lanes 4e + i/4 (e = 0..3); lane
// 4e + q points at row (base + e), columns 4q .. 4q + 3 of its group.
template <int D>
__device__ __forceinline__ bf16x8 tile_tr8(const u32x4* t, int r0, int c0, int lane) {
  const int r = r0 + 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int d = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  constexpr int ROWB = D * 2;
  const char* base = reinterpret_cast<const char*>(t);
  const char* p0 = base + r * ROWB + (((d >> 3) ^ swz_tile<D>(r)) << 4) + (d & 7) * 2;
  const char* p1 = base + (r + 8) * ROWB + (((d >> 3) ^ swz_tile<D>(r + 8)) << 4) + (d & 7) * 2;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)((__attribute__((address_space(3))) char*)p0));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)((__attribute__((address_space(3))) char*)p1));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Byte offset, inside a tile, of the transposed read that lane `lane` issues
// for tile_tr8-style operands of rows 0..15 (hi = 0: the rows 4h + (lane&15)/4,
// hi = 1: those + 8) and column block 0 (columns 0..31).  Column block m is
// at tr_offset ^ (m << 6) (the swizzle moves whole 64-byte groups in the
// same way for every m), rows 16 s further at + 16 s rows.  Adding a
// 256-byte aligned tile address keeps the XOR form valid.
template <int D>
__device__ __forceinline__ uint32_t tr_offset(int lane, int hi) {
  const int r = 4 * (lane >> 5) + ((lane & 15) >> 2) + 8 * hi;
  const int x = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int s = swz_tile<D>(r);
  return (uint32_t)(r * (D * 2) + ((s >> 2) << 6) + (((x ^ s) & 3) << 4) + 8 * (lane & 1));
}

__device__ __forceinline__ bf16x8 join_tr(u32x2 lo, u32x2 hi) {
  return __builtin_bit_cast(bf16x8, (u32x4){lo.x, lo.y, hi.x, hi.y});
}

// tile_tr8 operands for NS consecutive 16-row groups (rows 16 s .. past the
// addresses `lo`, `hi` built from tr_offset), issued and completed in one
// asm statement.  Through the builtin, the compiler would take each
// transposing read as possibly reading LDS that a global->LDS copy in
// flight is writing, and wait for every copy before it; these reads never
// touch the buffer being filled.
template <int D, int NS>
__device__ __forceinline__ void tile_tr8_asm(bf16x8 (&o)[NS], uint32_t lo, uint32_t hi) {
  constexpr int G = 16 * D * 2;  // bytes per 16-row group
  u32x2 r[2 * NS];
  if constexpr (NS == 2) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %5\n\t"
        "ds_read_b64_tr_b16 %2, %4 offset:%6\n\t"
        "ds_read_b64_tr_b16 %3, %5 offset:%6\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(lo), "v"(hi), "i"(G)
        : "memory");
  } else {
    static_assert(NS == 4, "2 or 4 row groups");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:%10\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%10\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:%11\n\t"
        "ds_read_b64_tr_b16 %5, %9 offset:%11\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %7, %9 offset:%12\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]),
          "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(lo), "v"(hi), "i"(G), "i"(2 * G), "i"(3 * G)
        : "memory");
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) o[s] = join_tr(r[2 * s], r[2 * s + 1]);
}

// Two 16-row groups for NM column blocks (block m at address ^ (m << 6)),
// all reads in one asm statement with one wait.
template <int D, int NM>
__device__ __forceinline__ void tile_tr8_asm_cols(bf16x8 (&o)[NM][2], uint32_t lo, uint32_t hi) {
  constexpr int G = 16 * D * 2;
  if constexpr (NM == 2) {
    u32x2 r[8];
    const uint32_t lo1 = lo ^ 64u, hi1 = hi ^ 64u;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%12\n\t"
        "ds_read_b64_tr_b16 %4, %10\n\t"
        "ds_read_b64_tr_b16 %5, %11\n\t"
        "ds_read_b64_tr_b16 %6, %10 offset:%12\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:%12\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]),
          "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(lo), "v"(hi), "v"(lo1), "v"(hi1), "i"(G)
        : "memory");
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int s = 0; s < 2; ++s) o[m][s] = join_tr(r[4 * m + 2 * s], r[4 * m + 2 * s + 1]);
  } else {
    static_assert(NM == 4, "2 or 4 column blocks");
    u32x2 r[16];
    const uint32_t lo1 = lo ^ 64u, hi1 = hi ^ 64u, lo2 = lo ^ 128u, hi2 = hi ^ 128u;
    const uint32_t lo3 = lo ^ 192u, hi3 = hi ^ 192u;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n\t"
        "ds_read_b64_tr_b16 %1, %17\n\t"
        "ds_read_b64_tr_b16 %2, %16 offset:%24\n\t"
        "ds_read_b64_tr_b16 %3, %17 offset:%24\n\t"
        "ds_read_b64_tr_b16 %4, %18\n\t"
        "ds_read_b64_tr_b16 %5, %19\n\t"
        "ds_read_b64_tr_b16 %6, %18 offset:%24\n\t"
        "ds_read_b64_tr_b16 %7, %19 offset:%24\n\t"
        "ds_read_b64_tr_b16 %8, %20\n\t"
        "ds_read_b64_tr_b16 %9, %21\n\t"
        "ds_read_b64_tr_b16 %10, %20 offset:%24\n\t"
        "ds_read_b64_tr_b16 %11, %21 offset:%24\n\t"
        "ds_read_b64_tr_b16 %12, %22\n\t"
        "ds_read_b64_tr_b16 %13, %23\n\t"
        "ds_read_b64_tr_b16 %14, %22 offset:%24\n\t"
        "ds_read_b64_tr_b16 %15, %23 offset:%24\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]),
          "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
          "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]),
          "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
        : "v"(lo), "v"(hi), "v"(lo1), "v"(hi1), "v"(lo2), "v"(hi2), "v"(lo3), "v"(hi3), "i"(G)
        : "memory");
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int s = 0; s < 2; ++s) o[m][s] = join_tr(r[4 * m + 2 * s], r[4 * m + 2 * s + 1]);
  }
}

}  // namespace vsa
