// attn_own_block.hip -- the own-block partial of leak-free causal MXFP8 attention, gfx950.
//
// TransformerEngine PR #3865, "Description", second bullet: each query's own 32-token block (at most
// 32 keys) is computed on a token-normalised copy of V (one power-of-two amplitude per token) and
// merged with the completed-block partial through the log-sum-exps. Reading used here: scores from
// the decoded rowwise MXFP8 Q/K (the operands the completed blocks use), softmax and P.V in fp32 with
// P not quantised, V decoded from the token-normalised codes.
//
// One workgroup per (b, hq, 32-query block): the block's Q, K and V rows are decoded once into LDS
// (the 32 queries share the same 32 keys), then 32x32 masked scores, a per-row softmax and the
// 32x128 output. HBM-bound: it reads 256 code bytes per query row and writes 516 bytes.
#include "device_common.h"
#include "launch.h"

namespace mxfa {

__global__ __launch_bounds__(256) void own_block_kernel(const uint8_t* __restrict__ qc, const uint8_t* __restrict__ qs,
                                                        const uint8_t* __restrict__ kc, const uint8_t* __restrict__ ks,
                                                        const uint8_t* __restrict__ vt,
                                                        const uint8_t* __restrict__ vta, int S, int Hq, int Hkv,
                                                        float scale, float* __restrict__ o,
                                                        float* __restrict__ lse) {
  __shared__ float Qm[32][129];
  __shared__ float Km[32][129];
  __shared__ float Vm[32][128];
  __shared__ float P[32][33];
  const int tid = threadIdx.x;
  const int cb = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int hk = hq / (Hq / Hkv);
  const int j0 = 32 * cb;
  const int64_t qrow0 = ((int64_t)b * Hq + hq) * S + j0;
  const int64_t krow0 = ((int64_t)b * Hkv + hk) * S + j0;
  for (int e = tid; e < 32 * 32; e += 256) {  // 4 code bytes per step
    const int r = e >> 5, d4 = (e & 31) * 4;
    const uint32_t cq = *reinterpret_cast<const uint32_t*>(qc + (qrow0 + r) * 128 + d4);
    const uint32_t ck = *reinterpret_cast<const uint32_t*>(kc + (krow0 + r) * 128 + d4);
    const uint32_t cv = *reinterpret_cast<const uint32_t*>(vt + (krow0 + r) * 128 + d4);
    const float sq = e8m0_to_f32(qs[(qrow0 + r) * 4 + (d4 >> 5)]);
    const float sk = e8m0_to_f32(ks[(krow0 + r) * 4 + (d4 >> 5)]);
    const float sv = e8m0_to_f32(vta[krow0 + r]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Qm[r][d4 + i] = e4m3_to_f32((cq >> (8 * i)) & 0xffu) * sq;
      Km[r][d4 + i] = e4m3_to_f32((ck >> (8 * i)) & 0xffu) * sk;
      Vm[r][d4 + i] = e4m3_to_f32((cv >> (8 * i)) & 0xffu) * sv;
    }
  }
  __syncthreads();
  {  // scores: thread -> (query i, four keys)
    const int i = tid >> 3, jg = (tid & 7) * 4;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = jg + jj;
      float acc = 0.f;
      for (int d = 0; d < 128; ++d) acc = fmaf(Qm[i][d], Km[j][d], acc);
      P[i][j] = (j <= i) ? acc * scale : -INFINITY;
    }
  }
  __syncthreads();
  if (tid < 32) {  // softmax of row i over keys 0..i
    const int i = tid;
    float m = -INFINITY;
    for (int j = 0; j <= i; ++j) m = fmaxf(m, P[i][j]);
    float l = 0.f;
    for (int j = 0; j < 32; ++j) {
      const float p = (j <= i) ? expf(P[i][j] - m) : 0.f;
      P[i][j] = p;
      l += p;
    }
    const float inv = 1.0f / l;
    for (int j = 0; j <= i; ++j) P[i][j] *= inv;
    lse[qrow0 + i] = m + logf(l);
  }
  __syncthreads();
  {  // output: thread -> (query i, 16 columns)
    const int i = tid >> 3, d0 = (tid & 7) * 16;
    float acc[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) acc[t] = 0.f;
    for (int j = 0; j <= i; ++j) {
      const float p = P[i][j];
#pragma unroll
      for (int t = 0; t < 16; ++t) acc[t] = fmaf(p, Vm[j][d0 + t], acc[t]);
    }
    float* dst = o + (qrow0 + i) * 128 + d0;
#pragma unroll
    for (int t = 0; t < 16; t += 4) *reinterpret_cast<float4*>(dst + t) = make_float4(acc[t], acc[t + 1], acc[t + 2], acc[t + 3]);
  }
}

hipError_t launch_attn_own_block(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                                 const uint8_t* vt, const uint8_t* vta, int B, int S, int Hq, int Hkv,
                                 float softmax_scale, float* o_o, float* lse_o, hipStream_t stream) {
  dim3 grid((unsigned)(S / 32), (unsigned)Hq, (unsigned)B);
  own_block_kernel<<<grid, dim3(256), 0, stream>>>(qc, qs, kc, ks, vt, vta, S, Hq, Hkv, softmax_scale, o_o, lse_o);
  return hipGetLastError();
}

}  // namespace mxfa
