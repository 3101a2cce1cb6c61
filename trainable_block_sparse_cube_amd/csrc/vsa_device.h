// Device-side helpers shared by the gfx950 kernels: element types, MFMA
// operand vectors, bf16 rounding and cross-lane exchanges.
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

// Key order used for V^T tiles ("MFMA order"): inside each group of 16 keys,
// storage position p holds key (p&3) + 8*((p>>2)&1) + 4*((p>>3)&1).  With
// it, the 8 keys a lane feeds to one 32x32x16 MFMA step of P*V are 16
// contiguous bytes.  The map is an involution on 0..15.
__device__ __host__ __forceinline__ int vt_key_of_pos(int p) {
  return (p & ~15) | (p & 3) | (((p >> 2) & 1) << 3) | (((p >> 3) & 1) << 2);
}

}  // namespace vsa
