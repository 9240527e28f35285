// launch.h -- host-side launchers of the libmxfa kernels (called by api.cpp after validation).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mxfa.h"

namespace mxfa {

// Workspace parts of the backward: decoded bf16 operands, head-major, and the transposed copies.
struct BwdWorkspace {
  uint16_t *qd, *qdt, *kd, *kdt, *vd, *gd, *gdt;  // [B,H,S,128] and [B,H,128,S]
  float* delta;                                     // [B,Hq,S]
  float* lse2;                                      // lse * log2(e), [B,Hq,S]
  size_t bytes;
};

// Size of the static device workspace of mxfa_attn_fwd_noalloc (noalloc.hip), as the header states it:
// 256 MiB, enough for the K and V encodings of B * Hkv * S <= 655360 (S = 32768 with 16 KV heads).
constexpr size_t kNoallocWorkspaceBytes = MXFA_NOALLOC_WORKSPACE_BYTES;
// That workspace's address on the current device (looked up once per device).
hipError_t noalloc_workspace(void** ptr);

hipError_t launch_quantize_rowwise(const uint16_t* x, int B, int S, int H, int64_t sb, int64_t ss, int64_t sh,
                                   uint8_t* codes, uint8_t* scales, hipStream_t stream);
hipError_t launch_quantize_v(const uint16_t* v, int B, int S, int H, int64_t sb, int64_t ss, int64_t sh,
                             uint8_t* col_codes, uint8_t* col_scales, uint8_t* tn_codes, uint8_t* tn_amps,
                             hipStream_t stream);
hipError_t launch_quantize_kv(const uint16_t* k, int64_t ksb, int64_t kss, int64_t ksh, const uint16_t* v,
                              int64_t vsb, int64_t vss, int64_t vsh, int B, int S, int H, uint8_t* kc, uint8_t* ks,
                              uint8_t* vc, uint8_t* vcs, uint8_t* vt, uint8_t* vta, hipStream_t stream);
hipError_t launch_attn_completed(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                                 const uint8_t* vc, const uint8_t* vcs, int B, int S, int Hq, int Hkv,
                                 float softmax_scale, float* o_c, float* lse_c, hipStream_t stream);
hipError_t launch_attn_fused(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                             const uint8_t* vc, const uint8_t* vcs, const uint8_t* vt, const uint8_t* vta, int B,
                             int S, int Hq, int Hkv, float softmax_scale, void* out, int64_t osb, int64_t oss,
                             int64_t osh, int out_bf16, float* lse_out, hipStream_t stream,
                             uint8_t* sf_o = nullptr,  // sf_o != null: MXFP8 O codes into out
                             const uint16_t* qbf = nullptr, int64_t qsb = 0, int64_t qss = 0,
                             int64_t qsh = 0);  // qbf != null: bf16 Q view, quantised in-kernel (qc, qs unused)
hipError_t launch_attn_leaky(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                             const uint8_t* vc, const uint8_t* vcs, int B, int S, int Hq, int Hkv, float softmax_scale,
                             void* out, int64_t osb, int64_t oss, int64_t osh, int out_bf16, float* lse_out,
                             hipStream_t stream);
hipError_t launch_attn_bwd(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                           const uint8_t* vt, const uint8_t* vta, const uint16_t* o, const float* lse,
                           const uint16_t* dout, int B, int S, int Hq, int Hkv, float softmax_scale, int64_t qsb,
                           int64_t qss, int64_t qsh, int64_t ksb, int64_t kss, int64_t ksh, const BwdWorkspace& ws,
                           uint16_t* dq, uint16_t* dk, uint16_t* dv, hipStream_t stream);
hipError_t launch_attn_own_block(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                                 const uint8_t* vt, const uint8_t* vta, int B, int S, int Hq, int Hkv,
                                 float softmax_scale, float* o_o, float* lse_o, hipStream_t stream);
hipError_t launch_lse_merge(const float* o_c, const float* lse_c, const float* o_o, const float* lse_o, int B, int S,
                            int H, void* out, int64_t osb, int64_t oss, int64_t osh, int out_bf16, float* lse_out,
                            hipStream_t stream);

}  // namespace mxfa
