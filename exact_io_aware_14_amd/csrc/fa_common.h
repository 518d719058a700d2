// Device-side helpers shared by the gfx950 attention kernels.
//
// Register layouts of the bf16 MFMA 32x32x16 instruction used throughout
// (wave64; lane l, half h = l / 32, column c = l % 32):
//   A operand (32 x 16, 8 bf16 per lane): row c, k-slots 8h .. 8h+7
//   B operand (16 x 32, 8 bf16 per lane): column c, k-slots 8h .. 8h+7
//   C/D accumulator (32 x 32, 16 fp32 per lane): column c, element r holds
//     row 8*(r/4) + 4h + (r%4).
// Which k a slot stands for never matters as long as the A and B operands of
// one instruction use the same slot-to-k assignment; the kernels choose that
// assignment so that an accumulator can be repacked as the next operand
// inside its own lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// Round two fp32 values to bf16 (nearest even) and pack them in one dword,
// the first value in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ uint4 as_u4(bf16x8 v) { return __builtin_bit_cast(uint4, v); }

// Eight consecutive elements of a row, as eight bf16 in a uint4. Storage
// type bf16 (uint16_t) is loaded as is; fp32 is rounded to nearest even.
// Rows past the end read as zeros.
template <typename T>
__device__ __forceinline__ uint4 load8(const T* p, bool valid);

template <>
__device__ __forceinline__ uint4 load8<uint16_t>(const uint16_t* p, bool valid) {
  uint4 z = {0u, 0u, 0u, 0u};
  return valid ? *reinterpret_cast<const uint4*>(p) : z;
}

template <>
__device__ __forceinline__ uint4 load8<float>(const float* p, bool valid) {
  uint4 r = {0u, 0u, 0u, 0u};
  if (valid) {
    float4 a = reinterpret_cast<const float4*>(p)[0];
    float4 b = reinterpret_cast<const float4*>(p)[1];
    r.x = pack_bf16x2(a.x, a.y);
    r.y = pack_bf16x2(a.z, a.w);
    r.z = pack_bf16x2(b.x, b.y);
    r.w = pack_bf16x2(b.z, b.w);
  }
  return r;
}

// Flip the sign of eight packed bf16 values (exact).
__device__ __forceinline__ uint4 negate8(uint4 u) {
  u.x ^= 0x80008000u;
  u.y ^= 0x80008000u;
  u.z ^= 0x80008000u;
  u.w ^= 0x80008000u;
  return u;
}

// Value from the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace fa
