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
  // Q and K rows unpadded (52 KB in all, three workgroups per CU); float4 chunk x of Q row r sits in
  // slot x ^ (r & 7), of K row r in slot x ^ ((r >> 2) & 7): the eight Q rows (i) and the eight K rows
  // (4k + jj) that one wave reads at a time fall in different banks
  __shared__ __align__(16) float Qm[32][128];
  __shared__ __align__(16) float Km[32][128];
  __shared__ __align__(16) float Vm[32][128];
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
    // v_cvt_pk_f32_fp8 decodes two OCP E4M3 codes exactly (every code checked on gfx950)
    const auto q01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cq, false), q23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cq, true);
    const auto k01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)ck, false), k23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)ck, true);
    const auto v01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cv, false), v23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cv, true);
    *reinterpret_cast<float4*>(&Qm[r][4 * ((d4 >> 2) ^ (r & 7))]) =
        make_float4(q01[0] * sq, q01[1] * sq, q23[0] * sq, q23[1] * sq);
    *reinterpret_cast<float4*>(&Km[r][4 * ((d4 >> 2) ^ ((r >> 2) & 7))]) =
        make_float4(k01[0] * sk, k01[1] * sk, k23[0] * sk, k23[1] * sk);
    *reinterpret_cast<float4*>(&Vm[r][d4]) = make_float4(v01[0] * sv, v01[1] * sv, v23[0] * sv, v23[1] * sv);
  }
  __syncthreads();
  {  // scores: thread -> (query i, four keys), each dot product accumulated in order of d
    const int i = tid >> 3, jg = (tid & 7) * 4;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int d = 0; d < 128; d += 4) {
      const float4 qv = *reinterpret_cast<const float4*>(&Qm[i][4 * ((d >> 2) ^ (i & 7))]);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = jg + jj;
        const float4 kv = *reinterpret_cast<const float4*>(&Km[j][4 * ((d >> 2) ^ ((j >> 2) & 7))]);
        acc[jj] = fmaf(qv.x, kv.x, acc[jj]);
        acc[jj] = fmaf(qv.y, kv.y, acc[jj]);
        acc[jj] = fmaf(qv.z, kv.z, acc[jj]);
        acc[jj] = fmaf(qv.w, kv.w, acc[jj]);
      }
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = jg + jj;
      P[i][j] = (j <= i) ? acc[jj] * scale : -INFINITY;
    }
  }
  __syncthreads();
  {  // softmax of row i over keys 0..i: the row's eight consecutive lanes take four keys each
    const int i = tid >> 3, jg = (tid & 7) * 4;
    float v[4];
    float m = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      v[jj] = P[i][jg + jj];  // -inf for keys after the query
      m = fmaxf(m, v[jj]);
    }
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    float l = 0.f;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      v[jj] = (jg + jj <= i) ? expf(v[jj] - m) : 0.f;
      l += v[jj];
    }
    l += __shfl_xor(l, 1);
    l += __shfl_xor(l, 2);
    l += __shfl_xor(l, 4);
    const float inv = 1.0f / l;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) P[i][jg + jj] = v[jj] * inv;
    if ((tid & 7) == 0) lse[qrow0 + i] = m + logf(l);
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
