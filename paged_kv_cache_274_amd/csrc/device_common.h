// Device helpers shared by the gfx950 kernels of libpkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlock = 16;      // tokens per physical KV block
constexpr int kWave = 64;       // CDNA wavefront width

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// bf16 storage type: raw 16-bit pattern.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16lo_to_f32(uint32_t packed) {
  return __uint_as_float(packed << 16);
}
__device__ __forceinline__ float bf16hi_to_f32(uint32_t packed) {
  return __uint_as_float(packed & 0xffff0000u);
}

// fp32 -> bf16 with round-to-nearest-even (gfx950 v_cvt_pk_bf16_f32); NaN
// stays NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Lane permutations inside a row of 16 lanes through DPP (no LDS traffic).
// quad_perm [1,0,3,2] = lane ^ 1; [2,3,0,1] = lane ^ 2; row_half_mirror maps
// lane i to 7 - i inside each half-row; row_mirror maps lane i to 15 - i;
// row_ror:n rotates the 16 lanes of a row by n.
enum : int {
  kDppXor1 = 0xB1,
  kDppXor2 = 0x4E,
  kDppRowHalfMirror = 0x141,
  kDppRowMirror = 0x140,
  kDppRowRor4 = 0x124,
  kDppRowRor8 = 0x128,
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of N consecutive lanes (N in 1, 2, 4, 8, 16); every
// lane of a group receives the group total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
  return x;
}

// Cross-row exchanges on VALU (gfx950 v_permlane16_swap / v_permlane32_swap):
// with both operands equal to x, the two results hold x of lane l and of lane
// l ^ 16 (resp. l ^ 32), so their sum or max is the pairwise combine.
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Combine lanes that share (lane mod N) across the whole wave, N in 4, 8, 16,
// 32, 64: every lane receives the sum (max) over the 64/N lanes of its class.
template <int N>
__device__ __forceinline__ float class_sum(float x) {
  if constexpr (N <= 4) x += dpp<kDppRowRor4>(x);
  if constexpr (N <= 8) x += dpp<kDppRowRor8>(x);
  if constexpr (N <= 16) x = xor16_sum(x);
  if constexpr (N <= 32) x = xor32_sum(x);
  return x;
}

template <int N>
__device__ __forceinline__ float class_max(float x) {
  if constexpr (N <= 4) x = fmaxf(x, dpp<kDppRowRor4>(x));
  if constexpr (N <= 8) x = fmaxf(x, dpp<kDppRowRor8>(x));
  if constexpr (N <= 16) x = xor16_max(x);
  if constexpr (N <= 32) x = xor32_max(x);
  return x;
}

// Sum and max over all 64 lanes.
__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);
  return class_sum<16>(x);
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp<kDppRowMirror>(x));
  return class_max<16>(x);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave-uniform copies of values the compiler cannot prove uniform (results of
// cross-lane shuffles), so that branches on them stay scalar.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform(int64_t x) {
  const uint64_t u = (uint64_t)x;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Read-only metadata (block tables, context lengths) viewed through the
// constant address space: with a wave-uniform index the load is a scalar
// load, counted apart from the vector loads of K and V, so waiting for it
// never waits for K/V data in flight.
#define PKV_CONSTANT __attribute__((address_space(4)))
template <typename T>
__device__ __forceinline__ const PKV_CONSTANT T* constant_view(const T* p) {
  return (const PKV_CONSTANT T*)p;
}

}  // namespace pkv
