// lse_merge.hip -- merge of the completed-block and own-block partials through their log-sum-exps
// (TransformerEngine PR #3865, "Description", second bullet), gfx950.
//
// Per row: M = max(lse_c, lse_o), w = e^(lse - M), O = (w_c O_c + w_o O_o) / (w_c + w_o),
// lse = M + ln(w_c + w_o); a row with no completed key has lse_c = -inf and w_c = 0. HBM-bound
// elementwise pass: 32 threads per D=128 row, 16-byte loads, output written through a strided
// [B,S,H,D] view as bf16 (round to nearest even) or fp32.
#include "device_common.h"
#include "launch.h"

namespace mxfa {

__global__ __launch_bounds__(256) void lse_merge_kernel(const float4* __restrict__ oc, const float* __restrict__ lc,
                                                        const float4* __restrict__ oo, const float* __restrict__ lo,
                                                        int S, int H, void* __restrict__ out, int64_t osb,
                                                        int64_t oss, int64_t osh, int out_bf16,
                                                        float* __restrict__ lse_out, int64_t nrows) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid >> 5;  // (b, h, s)
  const int part = (int)(gid & 31);
  if (row >= nrows) return;
  const int s = (int)(row % S);
  const int64_t bh = row / S;
  const int h = (int)(bh % H);
  const int b = (int)(bh / H);
  const float a = lc[row], c = lo[row];
  const float M = fmaxf(a, c);
  const float wc = (a == -INFINITY) ? 0.f : expf(a - M);
  const float wo = (c == -INFINITY) ? 0.f : expf(c - M);
  const float inv = 1.0f / (wc + wo);
  const float4 x = oc[row * 32 + part], y = oo[row * 32 + part];
  const float r0 = (wc * x.x + wo * y.x) * inv, r1 = (wc * x.y + wo * y.y) * inv;
  const float r2 = (wc * x.z + wo * y.z) * inv, r3 = (wc * x.w + wo * y.w) * inv;
  const int64_t off = b * osb + s * oss + h * osh + part * 4;
  if (out_bf16) {
    uint2 pk;
    pk.x = f32_to_bf16(r0) | (f32_to_bf16(r1) << 16);
    pk.y = f32_to_bf16(r2) | (f32_to_bf16(r3) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + off) = pk;
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + off) = make_float4(r0, r1, r2, r3);
  }
  if (part == 0 && lse_out) lse_out[row] = M + logf(wc + wo);
}

hipError_t launch_lse_merge(const float* o_c, const float* lse_c, const float* o_o, const float* lse_o, int B, int S,
                            int H, void* out, int64_t osb, int64_t oss, int64_t osh, int out_bf16, float* lse_out,
                            hipStream_t stream) {
  const int64_t nrows = (int64_t)B * H * S;
  const int64_t blocks = (nrows * 32 + 255) / 256;
  lse_merge_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
      reinterpret_cast<const float4*>(o_c), lse_c, reinterpret_cast<const float4*>(o_o), lse_o, S, H, out, osb, oss,
      osh, out_bf16, lse_out, nrows);
  return hipGetLastError();
}

}  // namespace mxfa
