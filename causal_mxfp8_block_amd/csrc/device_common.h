// device_common.h -- small gfx950 device helpers shared by the libmxfa kernels.
//
// MXFP8 here is E4M3 (OCP E4M3FN, largest finite value 448) element codes with one E8M0 byte per
// 32-element block, scale = 2^(byte - 127) (cudnn-frontend PR #1088, PR summary). The block
// exponent rule is the smallest k with amax <= 448 * 2^k, so no element ever saturates.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v2s __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float u2f(uint32_t x) { return __builtin_bit_cast(float, x); }

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return u2f(bits16 << 16); }

// E8M0 exponent of a block whose largest magnitude is `amax` (finite, >= 0), from its fp32 bits:
// amax = f * 2^E with f in [1, 2): k = E - 8 when f <= 1.75 (mantissa field <= 0x600000), else
// E - 7. Zero and fp32-subnormal maxima give E <= -127 and clamp to k = -127.
__device__ __forceinline__ int e8m0_exponent(float amax) {
  uint32_t u = f2u(amax) & 0x7fffffffu;
  int e = (int)(u >> 23);
  int k = e - 127 - 8 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
  k = (e == 0) ? -127 : k;
  return k < -127 ? -127 : k;
}

// 2^-k as an fp32 value for k in [-127, 127] (always a normal number: exponent field 127 - k >= 0
// only for k <= 127; k = 127 would give the subnormal 2^-127, which never occurs for bf16 or fp32
// block maxima, whose k is at most 120).
__device__ __forceinline__ float pow2_neg(int k) { return u2f((uint32_t)(127 - k) << 23); }

// Four fp32 values -> four E4M3 codes packed little-endian into one dword. Inputs must satisfy
// |x| <= 448 (the conversion does not saturate; the scale rule guarantees the bound).
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// E4M3 code -> fp32 value (exact), from the bit layout: exponent 0 is subnormal (m * 2^-9).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag = (e == 0) ? (float)m * 0x1p-9f : u2f(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

// E8M0 byte -> 2^(byte - 127) as fp32 (byte 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t byte) {
  return byte == 0 ? 0x1p-127f : u2f(byte << 23);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  uint32_t u = f2u(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace mxfa
