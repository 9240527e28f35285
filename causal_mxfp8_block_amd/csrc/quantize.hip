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

// One thread encodes one 32-element block (its four 16-byte loads in flight together), 4 threads a
// D=128 row (9.6 us for K at 16/4 heads, S = 32K, against 11.0 with one thread per 8 elements).
__device__ __forceinline__ void rowwise_group(const uint16_t* __restrict__ x, int S, int H, int64_t sb, int64_t ss,
                                              int64_t sh, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                              int64_t nrows, int64_t group) {
  const int64_t gid = group * 256 + threadIdx.x;
  const int64_t row = gid >> 2;  // input row order (b, s, h)
  const int part = (int)(gid & 3);
  if (row >= nrows) return;
  const int h = (int)(row % H);
  const int64_t bs = row / H;
  const int s = (int)(bs % S);
  const int b = (int)(bs / S);
  const uint4* src = reinterpret_cast<const uint4*>(x + b * sb + s * ss + h * sh + part * 32);
  uint4 raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[i] = src[i];
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = bf16_to_f32(w[j] & 0xffffu);
      v[8 * i + 2 * j + 1] = bf16_to_f32(w[j] >> 16);
      amax = fmaxf(amax, fmaxf(fabsf(v[8 * i + 2 * j]), fabsf(v[8 * i + 2 * j + 1])));
    }
  }
  const int k = e8m0_exponent(amax);
  const float m = pow2_neg(k);
  const int64_t orow = ((int64_t)b * H + h) * S + s;
  uint4 o[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    o[i].x = pack4_e4m3(v[16 * i] * m, v[16 * i + 1] * m, v[16 * i + 2] * m, v[16 * i + 3] * m);
    o[i].y = pack4_e4m3(v[16 * i + 4] * m, v[16 * i + 5] * m, v[16 * i + 6] * m, v[16 * i + 7] * m);
    o[i].z = pack4_e4m3(v[16 * i + 8] * m, v[16 * i + 9] * m, v[16 * i + 10] * m, v[16 * i + 11] * m);
    o[i].w = pack4_e4m3(v[16 * i + 12] * m, v[16 * i + 13] * m, v[16 * i + 14] * m, v[16 * i + 15] * m);
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + orow * 128 + part * 32);
  dst[0] = o[0];
  dst[1] = o[1];
  scales[orow * 4 + part] = (uint8_t)(k + 127);
}

__global__ __launch_bounds__(256) void quantize_rowwise_kernel(const uint16_t* __restrict__ x, int S, int H,
                                                               int64_t sb, int64_t ss, int64_t sh,
                                                               uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales, int64_t nrows) {
  rowwise_group(x, S, H, sb, ss, sh, codes, scales, nrows, blockIdx.x);
}

// One workgroup per (b, h, group of up to 64 tokens): the bf16 tile is staged in LDS once and read
// twice, by rows (token-normalised copy) and by columns (columnwise blocks). 64-token groups give
// twice the workgroups of 128-token ones, so that one group's loads overlap another's conversions and
// stores (16.4 to 13.0 us at 16/4 heads, S = 32K; 32-token groups: 15.4 us).
constexpr int VQ_TOK = 64;
constexpr int VQ_ROW = 128 + 8;  // bf16 elements per LDS row (padding spreads banks)

__device__ __forceinline__ void v_group(const uint16_t* __restrict__ v, int S, int H, int64_t sb, int64_t ss,
                                        int64_t sh, uint8_t* __restrict__ col_codes, uint8_t* __restrict__ col_scales,
                                        uint8_t* __restrict__ tn_codes, uint8_t* __restrict__ tn_amps,
                                        uint16_t* tile, int group, int h, int b) {
  const int tid = threadIdx.x;
  const int s0 = group * VQ_TOK;
  const int ntok = min(VQ_TOK, S - s0);  // a multiple of 32
  const int64_t bh = (int64_t)b * H + h;
  // Thread tid moves chunk tid % 16 of rows tid / 16 + 16 i: all its loads are issued before any is
  // waited for (rows past the last token re-read the last one; only rows < ntok are read back).
  constexpr int kLoads = VQ_TOK / 16;
  const int q = tid & 15;
  uint4 val[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int r = min((tid >> 4) + 16 * i, ntok - 1);
    val[i] = *reinterpret_cast<const uint4*>(v + b * sb + (int64_t)(s0 + r) * ss + h * sh + q * 8);
  }
#pragma unroll
  for (int i = 0; i < kLoads; ++i) *reinterpret_cast<uint4*>(tile + ((tid >> 4) + 16 * i) * VQ_ROW + q * 8) = val[i];
  __syncthreads();

  // Token-normalised copy: four threads per token, 32 elements each.
  if (tn_codes) {
    const int r = tid >> 2, part = tid & 3;
    if (r < ntok) {
      const uint16_t* src = tile + r * VQ_ROW + part * 32;
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(bf16_to_f32(src[i])));
      amax = fmaxf(amax, __shfl_xor(amax, 1));
      amax = fmaxf(amax, __shfl_xor(amax, 2));
      const int k = e8m0_exponent(amax);
      const float m = pow2_neg(k);
      uint8_t* dst = tn_codes + (bh * S + s0 + r) * 128 + part * 32;
#pragma unroll
      for (int i = 0; i < 32; i += 16) {
        uint4 o;
        o.x = pack4_e4m3(bf16_to_f32(src[i + 0]) * m, bf16_to_f32(src[i + 1]) * m, bf16_to_f32(src[i + 2]) * m,
                         bf16_to_f32(src[i + 3]) * m);
        o.y = pack4_e4m3(bf16_to_f32(src[i + 4]) * m, bf16_to_f32(src[i + 5]) * m, bf16_to_f32(src[i + 6]) * m,
                         bf16_to_f32(src[i + 7]) * m);
        o.z = pack4_e4m3(bf16_to_f32(src[i + 8]) * m, bf16_to_f32(src[i + 9]) * m, bf16_to_f32(src[i + 10]) * m,
                         bf16_to_f32(src[i + 11]) * m);
        o.w = pack4_e4m3(bf16_to_f32(src[i + 12]) * m, bf16_to_f32(src[i + 13]) * m, bf16_to_f32(src[i + 14]) * m,
                         bf16_to_f32(src[i + 15]) * m);
        *reinterpret_cast<uint4*>(dst + i) = o;
      }
      if (part == 0) tn_amps[bh * S + s0 + r] = (uint8_t)(k + 127);
    }
  }

  // Columnwise blocks: item = (d, u); two adjacent threads hold the two token blocks of one
  // column, so together they write 64 contiguous code bytes.
  if (col_codes) {
    const int nblk = ntok >> 5;
    for (int item = tid; item < 128 * 2; item += 256) {
      const int u = item & 1, d = item >> 1;
      if (u >= nblk) continue;
      float x[32];
      float amax = 0.f;
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        x[r] = bf16_to_f32(tile[(32 * u + r) * VQ_ROW + d]);
        amax = fmaxf(amax, fabsf(x[r]));
      }
      const int k = e8m0_exponent(amax);
      const float m = pow2_neg(k);
      uint8_t* dst = col_codes + (bh * 128 + d) * S + s0 + 32 * u;
#pragma unroll
      for (int r = 0; r < 32; r += 16) {
        uint4 o;
        o.x = pack4_e4m3(x[r + 0] * m, x[r + 1] * m, x[r + 2] * m, x[r + 3] * m);
        o.y = pack4_e4m3(x[r + 4] * m, x[r + 5] * m, x[r + 6] * m, x[r + 7] * m);
        o.z = pack4_e4m3(x[r + 8] * m, x[r + 9] * m, x[r + 10] * m, x[r + 11] * m);
        o.w = pack4_e4m3(x[r + 12] * m, x[r + 13] * m, x[r + 14] * m, x[r + 15] * m);
        *reinterpret_cast<uint4*>(dst + r) = o;
      }
      col_scales[(bh * (S / 32) + s0 / 32 + u) * 128 + d] = (uint8_t)(k + 127);
    }
  }
}

__global__ __launch_bounds__(256) void quantize_v_kernel(const uint16_t* __restrict__ v, int S, int H, int64_t sb,
                                                         int64_t ss, int64_t sh, uint8_t* __restrict__ col_codes,
                                                         uint8_t* __restrict__ col_scales,
                                                         uint8_t* __restrict__ tn_codes,
                                                         uint8_t* __restrict__ tn_amps) {
  __shared__ __align__(16) uint16_t tile[VQ_TOK * VQ_ROW];
  v_group(v, S, H, sb, ss, sh, col_codes, col_scales, tn_codes, tn_amps, tile, blockIdx.x, blockIdx.y, blockIdx.z);
}

// K (rowwise) and V (both forms) of one attention call in one launch, the bytes of the two kernels
// above: workgroups [0, nv) are V groups (token group g % ng, head (g / ng) % H, batch g / (ng H)),
// the V groups first since each moves more than a K workgroup; the rest are K workgroups. One
// dispatch instead of two, and the two encoders' workgroups share the machine.
__global__ __launch_bounds__(256) void quantize_kv_kernel(const uint16_t* __restrict__ k, int64_t ksb, int64_t kss,
                                                          int64_t ksh, const uint16_t* __restrict__ v, int64_t vsb,
                                                          int64_t vss, int64_t vsh, int S, int H, int ng, int64_t nv,
                                                          int64_t nrows, uint8_t* __restrict__ kc,
                                                          uint8_t* __restrict__ ks, uint8_t* __restrict__ vc,
                                                          uint8_t* __restrict__ vcs, uint8_t* __restrict__ vt,
                                                          uint8_t* __restrict__ vta) {
  __shared__ __align__(16) uint16_t tile[VQ_TOK * VQ_ROW];
  const int64_t g = blockIdx.x;
  if (g < nv) {
    const int gi = (int)(g % ng);
    const int64_t bh = g / ng;
    v_group(v, S, H, vsb, vss, vsh, vc, vcs, vt, vta, tile, gi, (int)(bh % H), (int)(bh / H));
  } else {
    rowwise_group(k, S, H, ksb, kss, ksh, kc, ks, nrows, g - nv);
  }
}

hipError_t launch_quantize_rowwise(const uint16_t* x, int B, int S, int H, int64_t sb, int64_t ss, int64_t sh,
                                   uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t nrows = (int64_t)B * S * H;
  const int64_t blocks = (nrows * 4 + 255) / 256;
  quantize_rowwise_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(x, S, H, sb, ss, sh, codes, scales,
                                                                             nrows);
  return hipGetLastError();
}

hipError_t launch_quantize_v(const uint16_t* v, int B, int S, int H, int64_t sb, int64_t ss, int64_t sh,
                             uint8_t* col_codes, uint8_t* col_scales, uint8_t* tn_codes, uint8_t* tn_amps,
                             hipStream_t stream) {
  dim3 grid((unsigned)((S + VQ_TOK - 1) / VQ_TOK), (unsigned)H, (unsigned)B);
  quantize_v_kernel<<<grid, dim3(256), 0, stream>>>(v, S, H, sb, ss, sh, col_codes, col_scales, tn_codes, tn_amps);
  return hipGetLastError();
}

hipError_t launch_quantize_kv(const uint16_t* k, int64_t ksb, int64_t kss, int64_t ksh, const uint16_t* v,
                              int64_t vsb, int64_t vss, int64_t vsh, int B, int S, int H, uint8_t* kc, uint8_t* ks,
                              uint8_t* vc, uint8_t* vcs, uint8_t* vt, uint8_t* vta, hipStream_t stream) {
  const int ng = (S + VQ_TOK - 1) / VQ_TOK;
  const int64_t nv = (int64_t)ng * H * B;
  const int64_t nrows = (int64_t)B * S * H;
  const int64_t nk = (nrows * 4 + 255) / 256;
  quantize_kv_kernel<<<dim3((unsigned)(nv + nk)), dim3(256), 0, stream>>>(k, ksb, kss, ksh, v, vsb, vss, vsh, S, H, ng,
                                                                         nv, nrows, kc, ks, vc, vcs, vt, vta);
  return hipGetLastError();
}

}  // namespace mxfa
