// api.cpp -- the C ABI of libmxfa.so (declared in include/mxfa.h): host-side validation, error
// reporting and launch of the gfx950 kernels. Nothing here computes on the host; every call either
// enqueues its kernels on the caller's stream or returns an error having enqueued nothing.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/mxfa.h"
#include "launch.h"

#define MXFA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The current device must be a gfx950; the answer is cached per device ordinal.
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(MXFA_ERR_NO_DEVICE, "no HIP device is available");
  }
  static std::mutex mu;
  static signed char ok[64];  // 0 unknown, 1 gfx950, -1 other
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= 64) return fail(MXFA_ERR_NO_DEVICE, "device ordinal %d out of range", dev);
  if (ok[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(MXFA_ERR_NO_DEVICE, "cannot query HIP device %d", dev);
    }
    ok[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    if (ok[dev] < 0) return fail(MXFA_ERR_NO_DEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  }
  if (ok[dev] < 0) return fail(MXFA_ERR_NO_DEVICE, "device %d is not gfx950", dev);
  return MXFA_OK;
}

// Largest sequence length: the attention kernels address one (b, head) slice of codes, S * 128 bytes,
// through a buffer resource whose record count is 32 bits, with 32-bit offsets inside it.
constexpr int kMaxS = 1 << 24;

int check_attn_shape(int B, int S, int Hq, int Hkv, int D) {
  if (D != 128) return fail(MXFA_ERR_UNSUPPORTED, "D = %d: only D = 128 is supported", D);
  if (B < 1 || S < 1 || Hq < 1 || Hkv < 1) return fail(MXFA_ERR_SHAPE, "B, S, Hq, Hkv must be >= 1");
  if (S > kMaxS) return fail(MXFA_ERR_SHAPE, "S = %d exceeds the largest supported length 2^24", S);
  if (S % 32 != 0) return fail(MXFA_ERR_SHAPE, "S = %d is not a multiple of 32", S);
  if (Hq % Hkv != 0) return fail(MXFA_ERR_SHAPE, "Hq = %d is not a multiple of Hkv = %d", Hq, Hkv);
  if ((int64_t)B * Hq > 65535 * 64 || Hq > 65535 || B > 65535 ||
      (int64_t)B * Hq * ((S + 127) / 128) > 0x7fffffff)
    return fail(MXFA_ERR_SHAPE, "B = %d, Hq = %d, S = %d exceed the launch grid", B, Hq, S);
  return MXFA_OK;
}

int check_view(const char* name, const void* p, int B, int S, int H, int64_t sb, int64_t ss, int64_t sh,
               int elem_align) {
  if (!p) return fail(MXFA_ERR_NULL, "%s is NULL", name);
  if (!aligned16(p)) return fail(MXFA_ERR_ALIGN, "%s is not 16-byte aligned", name);
  if (sb < 0 || ss < 0 || sh < 0) return fail(MXFA_ERR_SHAPE, "%s has a negative stride", name);
  if (sb % elem_align || ss % elem_align || sh % elem_align)
    return fail(MXFA_ERR_ALIGN, "%s strides (%lld, %lld, %lld) are not multiples of %d elements", name,
                (long long)sb, (long long)ss, (long long)sh, elem_align);
  // Rows of 128 elements must not overlap within one (b, s, h) grid point.
  if ((B > 1 && sb < 128) || (S > 1 && ss < 128) || (H > 1 && sh < 128))
    return fail(MXFA_ERR_SHAPE, "%s strides (%lld, %lld, %lld) overlap D = 128 rows", name, (long long)sb,
                (long long)ss, (long long)sh);
  return MXFA_OK;
}

int check_ptrs(const char* const* names, const void* const* ptrs, int n) {
  for (int i = 0; i < n; ++i) {
    if (!ptrs[i]) return fail(MXFA_ERR_NULL, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(MXFA_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
  }
  return MXFA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MXFA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MXFA_OK;
}

#define TRY(x)                 \
  do {                         \
    int st_ = (x);             \
    if (st_ != MXFA_OK) return st_; \
  } while (0)

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// attn_fwd's workspace: the K and V encodings (Q is quantised inside the attention kernel).
struct Workspace {
  uint8_t *kc, *ks, *vc, *vcs, *vt, *vta;
  size_t bytes;
};

Workspace carve(void* base, int B, int S, int Hq, int Hkv) {
  Workspace w{};
  const size_t nk = (size_t)B * Hkv * S;
  size_t off = 0;
  auto take = [&](size_t n) {
    uint8_t* p = base ? static_cast<uint8_t*>(base) + off : nullptr;
    off += align256(n);
    return p;
  };
  w.kc = take(nk * 128);
  w.ks = take(nk * 4);
  w.vc = take(nk * 128);
  w.vcs = take(nk * 4);
  w.vt = take(nk * 128);
  w.vta = take(nk);
  w.bytes = off;
  return w;
}

mxfa::BwdWorkspace carve_bwd(void* base, int B, int S, int Hq, int Hkv) {
  mxfa::BwdWorkspace w{};
  const size_t nq = (size_t)B * Hq * S * 128 * 2, nk = (size_t)B * Hkv * S * 128 * 2;
  size_t off = 0;
  auto take = [&](size_t n) {
    uint8_t* p = base ? static_cast<uint8_t*>(base) + off : nullptr;
    off += align256(n);
    return p;
  };
  w.qd = reinterpret_cast<uint16_t*>(take(nq));
  w.qdt = reinterpret_cast<uint16_t*>(take(nq));
  w.kd = reinterpret_cast<uint16_t*>(take(nk));
  w.kdt = reinterpret_cast<uint16_t*>(take(nk));
  w.vd = reinterpret_cast<uint16_t*>(take(nk));
  w.gd = reinterpret_cast<uint16_t*>(take(nq));
  w.gdt = reinterpret_cast<uint16_t*>(take(nq));
  w.delta = reinterpret_cast<float*>(take((size_t)B * Hq * S * 4));
  w.lse2 = reinterpret_cast<float*>(take((size_t)B * Hq * S * 4));
  w.bytes = off;
  return w;
}

}  // namespace

MXFA_EXPORT const char* mxfa_status_string(int status) {
  switch (status) {
    case MXFA_OK: return "ok";
    case MXFA_ERR_NULL: return "null pointer";
    case MXFA_ERR_SHAPE: return "invalid shape";
    case MXFA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MXFA_ERR_ALIGN: return "misaligned pointer or stride";
    case MXFA_ERR_NO_DEVICE: return "no gfx950 device";
    case MXFA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

MXFA_EXPORT const char* mxfa_last_error(void) { return g_last_error.c_str(); }

MXFA_EXPORT int mxfa_mxfp8_quantize(const void* x, int B, int S, int H, int D, int64_t sb, int64_t ss, int64_t sh,
                                    int mode, uint8_t* codes, uint8_t* scales, uint8_t* tn_codes, uint8_t* tn_amps,
                                    void* stream) {
  g_last_error.clear();
  if (D != 128) return fail(MXFA_ERR_UNSUPPORTED, "D = %d: only D = 128 is supported", D);
  if (B < 1 || S < 1 || H < 1) return fail(MXFA_ERR_SHAPE, "B, S, H must be >= 1");
  if (S > kMaxS) return fail(MXFA_ERR_SHAPE, "S = %d exceeds the largest supported length 2^24", S);
  if (B > 65535 || H > 65535) return fail(MXFA_ERR_SHAPE, "B = %d, H = %d exceed the launch grid", B, H);
  TRY(check_view("x", x, B, S, H, sb, ss, sh, 8));
  if (mode == MXFA_QUANT_ROWWISE) {
    const char* n[] = {"codes", "scales"};
    const void* p[] = {codes, scales};
    TRY(check_ptrs(n, p, 2));
    if (tn_codes || tn_amps) return fail(MXFA_ERR_UNSUPPORTED, "rowwise mode takes no token-normalised outputs");
    TRY(check_device());
    return hip_status(mxfa::launch_quantize_rowwise(static_cast<const uint16_t*>(x), B, S, H, sb, ss, sh, codes,
                                                    scales, static_cast<hipStream_t>(stream)),
                      "quantize_rowwise launch");
  }
  if (mode == MXFA_QUANT_V) {
    if (S % 32 != 0) return fail(MXFA_ERR_SHAPE, "S = %d is not a multiple of 32", S);
    const bool col = codes || scales, tn = tn_codes || tn_amps;
    if (!col && !tn) return fail(MXFA_ERR_NULL, "V mode needs the columnwise or the token-normalised outputs");
    if (col) {
      const char* n[] = {"codes", "scales"};
      const void* p[] = {codes, scales};
      TRY(check_ptrs(n, p, 2));
    }
    if (tn) {
      const char* n[] = {"tn_codes", "tn_amps"};
      const void* p[] = {tn_codes, tn_amps};
      TRY(check_ptrs(n, p, 2));
    }
    TRY(check_device());
    return hip_status(mxfa::launch_quantize_v(static_cast<const uint16_t*>(x), B, S, H, sb, ss, sh, codes, scales,
                                              tn_codes, tn_amps, static_cast<hipStream_t>(stream)),
                      "quantize_v launch");
  }
  return fail(MXFA_ERR_UNSUPPORTED, "unknown quantisation mode %d", mode);
}

MXFA_EXPORT int mxfa_mxfp8_quantize_kv(const void* k, int64_t ksb, int64_t kss, int64_t ksh, const void* v,
                                       int64_t vsb, int64_t vss, int64_t vsh, int B, int S, int H, int D,
                                       uint8_t* k_codes, uint8_t* k_scales, uint8_t* v_codes, uint8_t* v_scales,
                                       uint8_t* v_tn_codes, uint8_t* v_tn_amps, void* stream) {
  g_last_error.clear();
  if (D != 128) return fail(MXFA_ERR_UNSUPPORTED, "D = %d: only D = 128 is supported", D);
  if (B < 1 || S < 1 || H < 1) return fail(MXFA_ERR_SHAPE, "B, S, H must be >= 1");
  if (S > kMaxS) return fail(MXFA_ERR_SHAPE, "S = %d exceeds the largest supported length 2^24", S);
  if (S % 32 != 0) return fail(MXFA_ERR_SHAPE, "S = %d is not a multiple of 32", S);
  if (B > 65535 || H > 65535) return fail(MXFA_ERR_SHAPE, "B = %d, H = %d exceed the launch grid", B, H);
  TRY(check_view("k", k, B, S, H, ksb, kss, ksh, 8));
  TRY(check_view("v", v, B, S, H, vsb, vss, vsh, 8));
  const char* n[] = {"k_codes", "k_scales", "v_codes", "v_scales", "v_tn_codes", "v_tn_amps"};
  const void* p[] = {k_codes, k_scales, v_codes, v_scales, v_tn_codes, v_tn_amps};
  TRY(check_ptrs(n, p, 6));
  TRY(check_device());
  return hip_status(mxfa::launch_quantize_kv(static_cast<const uint16_t*>(k), ksb, kss, ksh,
                                             static_cast<const uint16_t*>(v), vsb, vss, vsh, B, S, H, k_codes, k_scales,
                                             v_codes, v_scales, v_tn_codes, v_tn_amps, static_cast<hipStream_t>(stream)),
                    "quantize_kv launch");
}

MXFA_EXPORT int mxfa_attn_fwd_completed_blocks(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc,
                                               const uint8_t* ks, const uint8_t* vc, const uint8_t* vcs, int B,
                                               int S, int Hq, int Hkv, int D, float softmax_scale, float* o_c,
                                               float* lse_c, void* stream) {
  g_last_error.clear();
  TRY(check_attn_shape(B, S, Hq, Hkv, D));
  const char* n[] = {"qc", "qs", "kc", "ks", "vc", "vcs", "o_c", "lse_c"};
  const void* p[] = {qc, qs, kc, ks, vc, vcs, o_c, lse_c};
  TRY(check_ptrs(n, p, 8));
  TRY(check_device());
  return hip_status(mxfa::launch_attn_completed(qc, qs, kc, ks, vc, vcs, B, S, Hq, Hkv, softmax_scale, o_c, lse_c,
                                                static_cast<hipStream_t>(stream)),
                    "attn_fwd_completed_blocks launch");
}

MXFA_EXPORT int mxfa_attn_fwd_own_block(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                                        const uint8_t* vt, const uint8_t* vta, int B, int S, int Hq, int Hkv, int D,
                                        float softmax_scale, float* o_o, float* lse_o, void* stream) {
  g_last_error.clear();
  TRY(check_attn_shape(B, S, Hq, Hkv, D));
  const char* n[] = {"qc", "qs", "kc", "ks", "vt", "vta", "o_o", "lse_o"};
  const void* p[] = {qc, qs, kc, ks, vt, vta, o_o, lse_o};
  TRY(check_ptrs(n, p, 8));
  TRY(check_device());
  return hip_status(mxfa::launch_attn_own_block(qc, qs, kc, ks, vt, vta, B, S, Hq, Hkv, softmax_scale, o_o, lse_o,
                                                static_cast<hipStream_t>(stream)),
                    "attn_fwd_own_block launch");
}

MXFA_EXPORT int mxfa_lse_merge(const float* o_c, const float* lse_c, const float* o_o, const float* lse_o, int B,
                               int S, int H, int D, void* out, int64_t osb, int64_t oss, int64_t osh, int out_dtype,
                               float* lse_out, void* stream) {
  g_last_error.clear();
  if (D != 128) return fail(MXFA_ERR_UNSUPPORTED, "D = %d: only D = 128 is supported", D);
  if (B < 1 || S < 1 || H < 1) return fail(MXFA_ERR_SHAPE, "B, S, H must be >= 1");
  if (S > kMaxS) return fail(MXFA_ERR_SHAPE, "S = %d exceeds the largest supported length 2^24", S);
  if (out_dtype != MXFA_OUT_BF16 && out_dtype != MXFA_OUT_F32)
    return fail(MXFA_ERR_UNSUPPORTED, "unknown output dtype %d", out_dtype);
  const char* n[] = {"o_c", "lse_c", "o_o", "lse_o"};
  const void* p[] = {o_c, lse_c, o_o, lse_o};
  TRY(check_ptrs(n, p, 4));
  TRY(check_view("out", out, B, S, H, osb, oss, osh, out_dtype == MXFA_OUT_BF16 ? 8 : 4));
  if (lse_out && !aligned16(lse_out)) return fail(MXFA_ERR_ALIGN, "lse_out is not 16-byte aligned");
  TRY(check_device());
  return hip_status(mxfa::launch_lse_merge(o_c, lse_c, o_o, lse_o, B, S, H, out, osb, oss, osh,
                                           out_dtype == MXFA_OUT_BF16, lse_out, static_cast<hipStream_t>(stream)),
                    "lse_merge launch");
}

MXFA_EXPORT int mxfa_attn_fwd_fused(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                                    const uint8_t* vc, const uint8_t* vcs, const uint8_t* vt, const uint8_t* vta,
                                    int B, int S, int Hq, int Hkv, int D, float softmax_scale, void* out,
                                    int64_t osb, int64_t oss, int64_t osh, int out_dtype, float* lse_out,
                                    void* stream) {
  g_last_error.clear();
  TRY(check_attn_shape(B, S, Hq, Hkv, D));
  const char* n[] = {"qc", "qs", "kc", "ks", "vc", "vcs", "vt", "vta"};
  const void* p[] = {qc, qs, kc, ks, vc, vcs, vt, vta};
  TRY(check_ptrs(n, p, 8));
  if (out_dtype != MXFA_OUT_BF16 && out_dtype != MXFA_OUT_F32)
    return fail(MXFA_ERR_UNSUPPORTED, "unknown output dtype %d", out_dtype);
  TRY(check_view("out", out, B, S, Hq, osb, oss, osh, out_dtype == MXFA_OUT_BF16 ? 8 : 4));
  if (lse_out && !aligned16(lse_out)) return fail(MXFA_ERR_ALIGN, "lse_out is not 16-byte aligned");
  TRY(check_device());
  return hip_status(mxfa::launch_attn_fused(qc, qs, kc, ks, vc, vcs, vt, vta, B, S, Hq, Hkv, softmax_scale, out, osb,
                                            oss, osh, out_dtype == MXFA_OUT_BF16, lse_out,
                                            static_cast<hipStream_t>(stream)),
                    "attn_fwd_fused launch");
}

MXFA_EXPORT int mxfa_attn_fwd_fused_bf16q(const void* q, int64_t qsb, int64_t qss, int64_t qsh, const uint8_t* kc,
                                          const uint8_t* ks, const uint8_t* vc, const uint8_t* vcs, const uint8_t* vt,
                                          const uint8_t* vta, int B, int S, int Hq, int Hkv, int D,
                                          float softmax_scale, void* out, int64_t osb, int64_t oss, int64_t osh,
                                          int out_dtype, float* lse_out, void* stream) {
  g_last_error.clear();
  TRY(check_attn_shape(B, S, Hq, Hkv, D));
  TRY(check_view("q", q, B, S, Hq, qsb, qss, qsh, 8));
  const char* n[] = {"kc", "ks", "vc", "vcs", "vt", "vta"};
  const void* p[] = {kc, ks, vc, vcs, vt, vta};
  TRY(check_ptrs(n, p, 6));
  if (out_dtype != MXFA_OUT_BF16 && out_dtype != MXFA_OUT_F32)
    return fail(MXFA_ERR_UNSUPPORTED, "unknown output dtype %d", out_dtype);
  TRY(check_view("out", out, B, S, Hq, osb, oss, osh, out_dtype == MXFA_OUT_BF16 ? 8 : 4));
  if (lse_out && !aligned16(lse_out)) return fail(MXFA_ERR_ALIGN, "lse_out is not 16-byte aligned");
  TRY(check_device());
  return hip_status(mxfa::launch_attn_fused(nullptr, nullptr, kc, ks, vc, vcs, vt, vta, B, S, Hq, Hkv, softmax_scale,
                                            out, osb, oss, osh, out_dtype == MXFA_OUT_BF16, lse_out,
                                            static_cast<hipStream_t>(stream), nullptr,
                                            static_cast<const uint16_t*>(q), qsb, qss, qsh),
                    "attn_fwd_fused_bf16q launch");
}

MXFA_EXPORT int mxfa_attn_fwd_fused_mxfp8(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc,
                                          const uint8_t* ks, const uint8_t* vc, const uint8_t* vcs,
                                          const uint8_t* vt, const uint8_t* vta, int B, int S, int Hq, int Hkv,
                                          int D, float softmax_scale, uint8_t* o_codes, int64_t osb, int64_t oss,
                                          int64_t osh, uint8_t* sf_o, float* lse_out, void* stream) {
  g_last_error.clear();
  TRY(check_attn_shape(B, S, Hq, Hkv, D));
  const char* n[] = {"qc", "qs", "kc", "ks", "vc", "vcs", "vt", "vta", "sf_o"};
  const void* p[] = {qc, qs, kc, ks, vc, vcs, vt, vta, sf_o};
  TRY(check_ptrs(n, p, 9));
  TRY(check_view("o_codes", o_codes, B, S, Hq, osb, oss, osh, 16));
  if (lse_out && !aligned16(lse_out)) return fail(MXFA_ERR_ALIGN, "lse_out is not 16-byte aligned");
  TRY(check_device());
  return hip_status(mxfa::launch_attn_fused(qc, qs, kc, ks, vc, vcs, vt, vta, B, S, Hq, Hkv, softmax_scale, o_codes,
                                            osb, oss, osh, 0, lse_out, static_cast<hipStream_t>(stream), sf_o),
                    "attn_fwd_fused_mxfp8 launch");
}

MXFA_EXPORT int mxfa_attn_fwd_leaky(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                                    const uint8_t* vc, const uint8_t* vcs, int B, int S, int Hq, int Hkv, int D,
                                    float softmax_scale, void* out, int64_t osb, int64_t oss, int64_t osh,
                                    int out_dtype, float* lse_out, void* stream) {
  g_last_error.clear();
  TRY(check_attn_shape(B, S, Hq, Hkv, D));
  const char* n[] = {"qc", "qs", "kc", "ks", "vc", "vcs"};
  const void* p[] = {qc, qs, kc, ks, vc, vcs};
  TRY(check_ptrs(n, p, 6));
  if (out_dtype != MXFA_OUT_BF16 && out_dtype != MXFA_OUT_F32)
    return fail(MXFA_ERR_UNSUPPORTED, "unknown output dtype %d", out_dtype);
  TRY(check_view("out", out, B, S, Hq, osb, oss, osh, out_dtype == MXFA_OUT_BF16 ? 8 : 4));
  if (lse_out && !aligned16(lse_out)) return fail(MXFA_ERR_ALIGN, "lse_out is not 16-byte aligned");
  TRY(check_device());
  return hip_status(mxfa::launch_attn_leaky(qc, qs, kc, ks, vc, vcs, B, S, Hq, Hkv, softmax_scale, out, osb, oss, osh,
                                            out_dtype == MXFA_OUT_BF16, lse_out, static_cast<hipStream_t>(stream)),
                    "attn_fwd_leaky launch");
}

MXFA_EXPORT size_t mxfa_attn_fwd_workspace_bytes(int B, int S, int Hq, int Hkv, int D) {
  if (D != 128 || B < 1 || S < 1 || S > kMaxS || Hq < 1 || Hkv < 1) return 0;
  return carve(nullptr, B, S, Hq, Hkv).bytes;
}

MXFA_EXPORT int mxfa_attn_fwd(const void* q, int64_t qsb, int64_t qss, int64_t qsh, const void* k, int64_t ksb,
                              int64_t kss, int64_t ksh, const void* v, int64_t vsb, int64_t vss, int64_t vsh, int B,
                              int S, int Hq, int Hkv, int D, float softmax_scale, void* workspace,
                              size_t workspace_bytes, void* out, int64_t osb, int64_t oss, int64_t osh, int out_dtype,
                              float* lse_out, void* stream) {
  g_last_error.clear();
  TRY(check_attn_shape(B, S, Hq, Hkv, D));
  TRY(check_view("q", q, B, S, Hq, qsb, qss, qsh, 8));
  TRY(check_view("k", k, B, S, Hkv, ksb, kss, ksh, 8));
  TRY(check_view("v", v, B, S, Hkv, vsb, vss, vsh, 8));
  if (out_dtype != MXFA_OUT_BF16 && out_dtype != MXFA_OUT_F32)
    return fail(MXFA_ERR_UNSUPPORTED, "unknown output dtype %d", out_dtype);
  TRY(check_view("out", out, B, S, Hq, osb, oss, osh, out_dtype == MXFA_OUT_BF16 ? 8 : 4));
  if (lse_out && !aligned16(lse_out)) return fail(MXFA_ERR_ALIGN, "lse_out is not 16-byte aligned");
  if (!workspace) return fail(MXFA_ERR_NULL, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(MXFA_ERR_ALIGN, "workspace is not 256-byte aligned");
  const Workspace w = carve(workspace, B, S, Hq, Hkv);
  if (workspace_bytes < w.bytes)
    return fail(MXFA_ERR_UNSUPPORTED, "workspace has %zu bytes, %zu needed", workspace_bytes, w.bytes);
  TRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint16_t *q16 = static_cast<const uint16_t*>(q), *k16 = static_cast<const uint16_t*>(k),
                 *v16 = static_cast<const uint16_t*>(v);
  TRY(hip_status(mxfa::launch_quantize_kv(k16, ksb, kss, ksh, v16, vsb, vss, vsh, B, S, Hkv, w.kc, w.ks, w.vc, w.vcs,
                                          w.vt, w.vta, st),
                 "quantize k and v"));
  return hip_status(mxfa::launch_attn_fused(nullptr, nullptr, w.kc, w.ks, w.vc, w.vcs, w.vt, w.vta, B, S, Hq, Hkv,
                                           softmax_scale, out, osb, oss, osh, out_dtype == MXFA_OUT_BF16, lse_out,
                                           st, nullptr, q16, qsb, qss, qsh),
                    "fused attention");
}

MXFA_EXPORT int mxfa_attn_fwd_noalloc(const void* q, int64_t qsb, int64_t qss, int64_t qsh, const void* k,
                                      int64_t ksb, int64_t kss, int64_t ksh, const void* v, int64_t vsb, int64_t vss,
                                      int64_t vsh, int B, int S, int Hq, int Hkv, int D, float softmax_scale,
                                      void* out, int64_t osb, int64_t oss, int64_t osh, int out_dtype,
                                      float* lse_out, void* stream) {
  g_last_error.clear();
  TRY(check_attn_shape(B, S, Hq, Hkv, D));
  TRY(check_view("q", q, B, S, Hq, qsb, qss, qsh, 8));
  TRY(check_view("k", k, B, S, Hkv, ksb, kss, ksh, 8));
  TRY(check_view("v", v, B, S, Hkv, vsb, vss, vsh, 8));
  if (out_dtype != MXFA_OUT_BF16 && out_dtype != MXFA_OUT_F32)
    return fail(MXFA_ERR_UNSUPPORTED, "unknown output dtype %d", out_dtype);
  TRY(check_view("out", out, B, S, Hq, osb, oss, osh, out_dtype == MXFA_OUT_BF16 ? 8 : 4));
  if (lse_out && !aligned16(lse_out)) return fail(MXFA_ERR_ALIGN, "lse_out is not 16-byte aligned");
  const size_t need = carve(nullptr, B, S, Hq, Hkv).bytes;
  if (need > mxfa::kNoallocWorkspaceBytes)
    return fail(MXFA_ERR_UNSUPPORTED, "B = %d, S = %d, Hkv = %d need %zu workspace bytes; the static workspace holds %zu",
                B, S, Hkv, need, mxfa::kNoallocWorkspaceBytes);
  TRY(check_device());
  void* ws = nullptr;
  TRY(hip_status(mxfa::noalloc_workspace(&ws), "static workspace address"));
  const Workspace w = carve(ws, B, S, Hq, Hkv);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint16_t *q16 = static_cast<const uint16_t*>(q), *k16 = static_cast<const uint16_t*>(k),
                 *v16 = static_cast<const uint16_t*>(v);
  TRY(hip_status(mxfa::launch_quantize_kv(k16, ksb, kss, ksh, v16, vsb, vss, vsh, B, S, Hkv, w.kc, w.ks, w.vc, w.vcs,
                                          w.vt, w.vta, st),
                 "quantize k and v"));
  return hip_status(mxfa::launch_attn_fused(nullptr, nullptr, w.kc, w.ks, w.vc, w.vcs, w.vt, w.vta, B, S, Hq, Hkv,
                                           softmax_scale, out, osb, oss, osh, out_dtype == MXFA_OUT_BF16, lse_out,
                                           st, nullptr, q16, qsb, qss, qsh),
                    "fused attention");
}

MXFA_EXPORT size_t mxfa_attn_bwd_workspace_bytes(int B, int S, int Hq, int Hkv, int D) {
  if (D != 128 || B < 1 || S < 1 || S > kMaxS || Hq < 1 || Hkv < 1) return 0;
  return carve_bwd(nullptr, B, S, Hq, Hkv).bytes;
}

MXFA_EXPORT int mxfa_attn_bwd(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                              const uint8_t* vt, const uint8_t* vta, const void* o, const float* lse, const void* dout,
                              int B, int S, int Hq, int Hkv, int D, float softmax_scale, int64_t qsb, int64_t qss,
                              int64_t qsh, int64_t ksb, int64_t kss, int64_t ksh, void* workspace,
                              size_t workspace_bytes, void* dq, void* dk, void* dv, void* stream) {
  g_last_error.clear();
  TRY(check_attn_shape(B, S, Hq, Hkv, D));
  const char* n[] = {"qc", "qs", "kc", "ks", "vt", "vta", "lse"};
  const void* p[] = {qc, qs, kc, ks, vt, vta, lse};
  TRY(check_ptrs(n, p, 7));
  TRY(check_view("o", o, B, S, Hq, qsb, qss, qsh, 8));
  TRY(check_view("dout", dout, B, S, Hq, qsb, qss, qsh, 8));
  TRY(check_view("dq", dq, B, S, Hq, qsb, qss, qsh, 8));
  TRY(check_view("dk", dk, B, S, Hkv, ksb, kss, ksh, 8));
  TRY(check_view("dv", dv, B, S, Hkv, ksb, kss, ksh, 8));
  if (!workspace) return fail(MXFA_ERR_NULL, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(MXFA_ERR_ALIGN, "workspace is not 256-byte aligned");
  const mxfa::BwdWorkspace w = carve_bwd(workspace, B, S, Hq, Hkv);
  if (workspace_bytes < w.bytes)
    return fail(MXFA_ERR_UNSUPPORTED, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
                w.bytes);
  TRY(check_device());
  return hip_status(mxfa::launch_attn_bwd(qc, qs, kc, ks, vt, vta, static_cast<const uint16_t*>(o), lse,
                                          static_cast<const uint16_t*>(dout), B, S, Hq, Hkv, softmax_scale, qsb, qss,
                                          qsh, ksb, kss, ksh, w, static_cast<uint16_t*>(dq),
                                          static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv),
                                          static_cast<hipStream_t>(stream)),
                    "attn_bwd launch");
}

