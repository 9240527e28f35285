// quantize.hip -- MXFP8 quantisers for Q/K (rowwise along D) and V (columnwise over 32 tokens plus
// the token-normalised copy), gfx950.
//
// TransformerEngine PR #3865, "Description": P.V contracts over tokens, so V's MXFP8 scale is shared
// by 32 consecutive tokens of one head-dim column; the own block reads a token-normalised V copy
// with one power-of-two amplitude per token; Q/K are "rowwise MXFP8 bytes" (blocks of 32 along D).
// Every block: E8M0 exponent k = least k with amax <= 448 * 2^k, codes = E4M3(x * 2^-k).
//
// Both kernels are HBM-bound codecs: one pass over the bf16 input, 16-byte loads, each output
// written once.
#include "device_common.h"
#include "launch.h"

namespace mxfa {

// One thread encodes 8 consecutive elements; 4 threads form a 32-element block, 16 a D=128 row.
__global__ __launch_bounds__(256) void quantize_rowwise_kernel(const uint16_t* __restrict__ x, int S, int H,
                                                               int64_t sb, int64_t ss, int64_t sh,
                                                               uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales, int64_t nrows) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid >> 4;  // input row order (b, s, h)
  const int part = (int)(gid & 15);
  if (row >= nrows) return;  // whole 16-lane rows leave together
  const int h = (int)(row % H);
  const int64_t bs = row / H;
  const int s = (int)(bs % S);
  const int b = (int)(bs / S);
  const uint4 raw = *reinterpret_cast<const uint4*>(x + b * sb + s * ss + h * sh + part * 8);
  float v[8];
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(w[i] & 0xffffu);
    v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int k = e8m0_exponent(amax);
  const float m = pow2_neg(k);
  uint2 out;
  out.x = pack4_e4m3(v[0] * m, v[1] * m, v[2] * m, v[3] * m);
  out.y = pack4_e4m3(v[4] * m, v[5] * m, v[6] * m, v[7] * m);
  const int64_t orow = ((int64_t)b * H + h) * S + s;
  *reinterpret_cast<uint2*>(codes + orow * 128 + part * 8) = out;
  if ((part & 3) == 0) scales[orow * 4 + (part >> 2)] = (uint8_t)(k + 127);
}

// One wave per (b, h, 32-token block): the bf16 block is staged in LDS once and read twice, by rows
// (token-normalised copy) and by columns (the columnwise block of each head-dim column). Small
// single-wave workgroups keep many blocks in different phases at once, so HBM reads and writes
// overlap across them.
constexpr int VQ_TOK = 32;
constexpr int VQ_ROW = 128 + 8;  // bf16 elements per LDS row (padding spreads banks)

__global__ __launch_bounds__(64) void quantize_v_kernel(const uint16_t* __restrict__ v, int S, int H, int64_t sb,
                                                        int64_t ss, int64_t sh, uint8_t* __restrict__ col_codes,
                                                        uint8_t* __restrict__ col_scales,
                                                        uint8_t* __restrict__ tn_codes,
                                                        uint8_t* __restrict__ tn_amps) {
  __shared__ __align__(16) uint16_t tile[VQ_TOK * VQ_ROW];
  const int lane = threadIdx.x;
  const int s0 = blockIdx.x * VQ_TOK, h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * H + h;
  // 32 rows x 16 chunks of 16 bytes: lane takes chunks lane + 64 i, four whole rows per instruction
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = lane + 64 * i, r = c >> 4, q = c & 15;
    const uint4 val = *reinterpret_cast<const uint4*>(v + b * sb + (int64_t)(s0 + r) * ss + h * sh + q * 8);
    *reinterpret_cast<uint4*>(tile + r * VQ_ROW + q * 8) = val;
  }
  __syncthreads();

  // Token-normalised copy: two lanes per token, 64 elements each.
  if (tn_codes) {
    const int r = lane >> 1, half = lane & 1;
    const uint16_t* src = tile + r * VQ_ROW + half * 64;
    float x[64];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 w = *reinterpret_cast<const uint4*>(src + 8 * i);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * i + 2 * j] = bf16_to_f32(ww[j] & 0xffffu);
        x[8 * i + 2 * j + 1] = bf16_to_f32(ww[j] >> 16);
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    const int k = e8m0_exponent(amax);
    const float m = pow2_neg(k);
    uint8_t* dst = tn_codes + (bh * S + s0 + r) * 128 + half * 64;
#pragma unroll
    for (int i = 0; i < 64; i += 16) {
      uint4 o;
      o.x = pack4_e4m3(x[i + 0] * m, x[i + 1] * m, x[i + 2] * m, x[i + 3] * m);
      o.y = pack4_e4m3(x[i + 4] * m, x[i + 5] * m, x[i + 6] * m, x[i + 7] * m);
      o.z = pack4_e4m3(x[i + 8] * m, x[i + 9] * m, x[i + 10] * m, x[i + 11] * m);
      o.w = pack4_e4m3(x[i + 12] * m, x[i + 13] * m, x[i + 14] * m, x[i + 15] * m);
      *reinterpret_cast<uint4*>(dst + i) = o;
    }
    if (half == 0) tn_amps[bh * S + s0 + r] = (uint8_t)(k + 127);
  }

  // Columnwise block of the 32 tokens: lane takes columns d = 2 lane and 2 lane + 1, reading one dword
  // (both columns) per row, so each row read is 256 contiguous bytes across the wave.
  if (col_codes) {
    float x0[32], x1[32];
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(tile + r * VQ_ROW + 2 * lane);
      x0[r] = bf16_to_f32(w & 0xffffu);
      x1[r] = bf16_to_f32(w >> 16);
      a0 = fmaxf(a0, fabsf(x0[r]));
      a1 = fmaxf(a1, fabsf(x1[r]));
    }
    const int k0 = e8m0_exponent(a0), k1 = e8m0_exponent(a1);
    const float m0 = pow2_neg(k0), m1 = pow2_neg(k1);
    uint8_t* dst0 = col_codes + (bh * 128 + 2 * lane) * S + s0;
    uint8_t* dst1 = dst0 + S;
#pragma unroll
    for (int r = 0; r < 32; r += 16) {
      uint4 o0, o1;
      o0.x = pack4_e4m3(x0[r + 0] * m0, x0[r + 1] * m0, x0[r + 2] * m0, x0[r + 3] * m0);
      o0.y = pack4_e4m3(x0[r + 4] * m0, x0[r + 5] * m0, x0[r + 6] * m0, x0[r + 7] * m0);
      o0.z = pack4_e4m3(x0[r + 8] * m0, x0[r + 9] * m0, x0[r + 10] * m0, x0[r + 11] * m0);
      o0.w = pack4_e4m3(x0[r + 12] * m0, x0[r + 13] * m0, x0[r + 14] * m0, x0[r + 15] * m0);
      o1.x = pack4_e4m3(x1[r + 0] * m1, x1[r + 1] * m1, x1[r + 2] * m1, x1[r + 3] * m1);
      o1.y = pack4_e4m3(x1[r + 4] * m1, x1[r + 5] * m1, x1[r + 6] * m1, x1[r + 7] * m1);
      o1.z = pack4_e4m3(x1[r + 8] * m1, x1[r + 9] * m1, x1[r + 10] * m1, x1[r + 11] * m1);
      o1.w = pack4_e4m3(x1[r + 12] * m1, x1[r + 13] * m1, x1[r + 14] * m1, x1[r + 15] * m1);
      *reinterpret_cast<uint4*>(dst0 + r) = o0;
      *reinterpret_cast<uint4*>(dst1 + r) = o1;
    }
    *reinterpret_cast<uint16_t*>(col_scales + (bh * (S / 32) + s0 / 32) * 128 + 2 * lane) =
        (uint16_t)((k0 + 127) | ((k1 + 127) << 8));
  }
}

hipError_t launch_quantize_rowwise(const uint16_t* x, int B, int S, int H, int64_t sb, int64_t ss, int64_t sh,
                                   uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t nrows = (int64_t)B * S * H;
  const int64_t blocks = (nrows * 16 + 255) / 256;
  quantize_rowwise_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(x, S, H, sb, ss, sh, codes, scales,
                                                                             nrows);
  return hipGetLastError();
}

hipError_t launch_quantize_v(const uint16_t* v, int B, int S, int H, int64_t sb, int64_t ss, int64_t sh,
                             uint8_t* col_codes, uint8_t* col_scales, uint8_t* tn_codes, uint8_t* tn_amps,
                             hipStream_t stream) {
  dim3 grid((unsigned)(S / VQ_TOK), (unsigned)H, (unsigned)B);  // S % 32 == 0 (checked by the caller)
  quantize_v_kernel<<<grid, dim3(64), 0, stream>>>(v, S, H, sb, ss, sh, col_codes, col_scales, tn_codes, tn_amps);
  return hipGetLastError();
}

}  // namespace mxfa
