// mfma_peak.hip -- throughput probe of the block-scaled FP8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4)
// on the device, for the benchmark's "% of the measured peak": every wave runs four independent
// accumulation chains of the instruction the attention kernel uses, with no other work, two waves per
// SIMD. Built into libmxfa_peak.so, separate from the attention library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(512, 1) void mfma_peak_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 + lane;  // E4M3 codes near 1.0
    b[i] = 0x30303030 + i;
  }
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 127, 0, 127);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 0, 0, 0, 126, 0, 127);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 0, 0, 0, 125, 0, 127);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 0, 0, 0, 124, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

// Launches `blocks` workgroups of 8 waves (two per SIMD), each wave issuing 4 * iters MFMAs of
// 32 * 32 * 64 * 2 FLOP, on `stream`; out receives one float per thread (blocks * 512). Returns a
// hipError_t.
extern "C" __attribute__((visibility("default"))) int mxfa_peak_mfma_fp8(int blocks, int iters, float* out,
                                                                        void* stream) {
  if (blocks <= 0 || iters <= 0 || !out) return (int)hipErrorInvalidValue;
  mfma_peak_kernel<<<dim3(blocks), dim3(512), 0, static_cast<hipStream_t>(stream)>>>(iters, out);
  return (int)hipGetLastError();
}
