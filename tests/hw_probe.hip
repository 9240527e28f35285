// hw_probe.hip -- test-only gfx950 kernels that measure two hardware operations the attention kernel
// relies on, so that the tests can bound them against exact arithmetic on the host:
//
//  * probe_scores: S = Q K^T for MXFP8 operands (E4M3 codes, one E8M0 per 32 along D) on the
//    block-scaled FP8 MFMA v_mfma_scale_f32_32x32x64_f8f6f4, in the arrangement of the attention
//    kernel's scores: K is the A operand, Q the B operand, D = 128 contracted in two 64-wide steps
//    (the first into a zero accumulator, the second accumulating), lane (r, h) supplying bytes
//    d = 64m + 16h + [0,16) and 64m + 32 + 16h + [0,16) of its row with the scale of D-block 2m + h.
//    The accumulator is not rounded correctly by the hardware; the tests compare every score with
//    the exact dot product of the decoded operands.
//  * probe_cvt: fp32 -> E4M3 codes with v_cvt_pk_fp8_f32, four values per lane, the conversion the
//    attention kernel uses for P and for Q.
//
// Not part of libmxfa: built into tests/libhw_probe.so for the GPU tests only.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v8i load_operand(const uint8_t* row, int m, int h) {
  const uint4 a = *reinterpret_cast<const uint4*>(row + 64 * m + 16 * h);
  const uint4 b = *reinterpret_cast<const uint4*>(row + 64 * m + 32 + 16 * h);
  v8i r;
  r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
  r[4] = (int)b.x; r[5] = (int)b.y; r[6] = (int)b.z; r[7] = (int)b.w;
  return r;
}

// One wave per 32 x 32 block of scores: blockIdx.x is the key block, blockIdx.y the query block.
__global__ __launch_bounds__(64) void score_probe_kernel(const uint8_t* kc, const uint8_t* ks, const uint8_t* qc,
                                                         const uint8_t* qs, int nk, float* out) {
  const int lane = threadIdx.x, r = lane & 31, h = lane >> 5;
  const int key = blockIdx.x * 32 + r, query = blockIdx.y * 32 + r;
  const uint8_t* krow = kc + (int64_t)key * 128;
  const uint8_t* qrow = qc + (int64_t)query * 128;
  v16f acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const v8i a = load_operand(krow, m, h), b = load_operand(qrow, m, h);
    const int sa = ks[(int64_t)key * 4 + 2 * m + h], sb = qs[(int64_t)query * 4 + 2 * m + h];
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, sa, 0, sb);
  }
  // element i of lane (c, h): row (key) 8(i/4) + 4h + i%4 of the block, column (query) c
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int kk = blockIdx.x * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
    out[(int64_t)(blockIdx.y * 32 + r) * nk + kk] = acc[i];
  }
}

__global__ void cvt_probe_kernel(const float* x, int n4, uint32_t* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const float4 v = reinterpret_cast<const float4*>(x)[i];
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(v.x, v.y, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(v.z, v.w, w, true);
  out[i] = (uint32_t)w;
}

}  // namespace

// Scores of nq queries against nk keys (both multiples of 32): kc/qc codes [n][128], ks/qs scale
// bytes [n][4], out fp32 [nq][nk]. Device pointers; runs on the null stream. Returns a hipError_t.
extern "C" __attribute__((visibility("default"))) int probe_scores(const uint8_t* kc, const uint8_t* ks,
                                                                  const uint8_t* qc, const uint8_t* qs, int nk,
                                                                  int nq, float* out) {
  if (nk <= 0 || nq <= 0 || nk % 32 || nq % 32) return (int)hipErrorInvalidValue;
  score_probe_kernel<<<dim3(nk / 32, nq / 32), dim3(64)>>>(kc, ks, qc, qs, nk, out);
  return (int)hipGetLastError();
}

// E4M3 codes of n fp32 values (n a multiple of 4), four codes per output dword, the first in the
// lowest byte. Device pointers; null stream.
extern "C" __attribute__((visibility("default"))) int probe_cvt(const float* x, int n, uint32_t* out) {
  if (n <= 0 || n % 4) return (int)hipErrorInvalidValue;
  const int n4 = n / 4;
  cvt_probe_kernel<<<dim3((n4 + 255) / 256), dim3(256)>>>(x, n4, out);
  return (int)hipGetLastError();
}
