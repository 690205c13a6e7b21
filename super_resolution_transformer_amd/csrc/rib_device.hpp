// rib_device.hpp -- gfx950 device helpers shared by the library's kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rib {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (low half = a), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t r = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

// Two floats -> packed bf16 pair by truncation (the high 16 bits of each; low
// half = a): one v_perm_b32.
__device__ __forceinline__ uint32_t pack_bf16_trunc(float a, float b) {
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, a), 0x07060302u);
}

// float value of one bf16 half of a packed dword
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __builtin_bit_cast(float, x & 0xFFFF0000u); }

// Round a float to the nearest bf16 value (nearest even), returned as float.
__device__ __forceinline__ float round_bf16(float a) { return bf16_lo(pack_bf16(a, 0.0f)); }

// Values of lane l%32 and lane l%32+32, for every lane l (v_permlane32_swap).
struct LanePair {
  float lo, hi;
};
__device__ __forceinline__ LanePair lane_pair(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  return {__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])};
}

// Value held by lane l^1 (DPP quad permutation [1,0,3,2]).
__device__ __forceinline__ uint32_t lane_xor1(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
}

// 1/x on the reciprocal unit (v_rcp_f32, about 1 ulp) instead of the correctly rounded
// division this library is built with (about ten instructions): for the bf16 epilogues,
// which round their results to 8 significant bits.  x must be a normal number.
__device__ __forceinline__ float rcp_approx(float x) { return __builtin_amdgcn_rcpf(x); }

// logistic sigmoid for the bf16 epilogues: 1 + e^-z >= 1, so the reciprocal is in (0, 1]
__device__ __forceinline__ float sigmoidf(float z) { return rcp_approx(1.0f + __expf(-z)); }

// Map workgroup i of a launch of 8*per workgroups so that consecutive logical
// blocks run on the same XCD (the dispatcher sends block i to XCD i % 8).
__device__ __forceinline__ int xcd_swizzle(int bid, int grid) {
  const int per = grid >> 3;
  return (bid & 7) * per + (bid >> 3);
}

}  // namespace rib
