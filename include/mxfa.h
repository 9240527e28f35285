/*
 * mxfa.h -- C ABI of libmxfa.so: leak-free causal MXFP8 attention forward for AMD MI355X (gfx950).
 *
 * The method is TransformerEngine PR #3865, "[PyTorch] Add causal MXFP8 attention without
 * future-token leakage through V scales" (section "Description"): a columnwise MXFP8 V scale is
 * shared by 32 consecutive tokens, so under an ordinary causal mask a later token in a query's own
 * 32-token block can change how earlier visible V values round. Query i therefore splits its keys at
 * 32*floor(i/32): completed blocks run in MXFP8 with columnwise V scales that cover visible tokens
 * only; the query's own block (at most 32 keys) runs on a token-normalised V copy; the two partials
 * are merged through their log-sum-exps. MXFP8 means E4M3 element codes with one E8M0 power-of-two
 * scale per 32 elements along the contraction axis (cudnn-frontend PR #1088, PR summary).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is DEVICE memory owned by the caller. The library never allocates or
 *     frees memory, never copies between host and device and never synchronises: all work is
 *     enqueued on `stream` (a hipStream_t; NULL is the null stream) and runs asynchronously.
 *   - Every call validates its arguments on the host first. On any error it returns a nonzero
 *     mxfa_status, enqueues nothing, and mxfa_last_error() names the violated constraint. There is
 *     no slower fallback path for unsupported shapes.
 *   - Supported shapes: D == 128, S % 32 == 0, 1 <= S <= 2^24, B, H >= 1, Hq % Hkv == 0 (GQA: q-head
 *     hq reads kv-head hq / (Hq/Hkv)), equal query and key lengths, causal.
 *   - bf16 tensors are addressed by element strides (sb, ss, sh) of a logical [B,S,H,D] tensor with
 *     unit stride along D (BSHD and SBHD are both such views). Pointers must be 16-byte aligned and
 *     bf16 strides multiples of 8 elements.
 *   - Inputs must be finite and the scaled scores finite in fp32; non-finite values are outside the
 *     contract and are not checked.
 *   - Code/scale layouts (all row-major, bytes):
 *       Q/K rowwise codes   [B,H,S,D]      scales [B,H,S,D/32]   (E8M0 bytes, scale = 2^(byte-127))
 *       V columnwise codes  [B,H,D,S]      scales [B,H,S/32,D]   (keys contiguous per column)
 *       V token-normalised  [B,H,S,D]      amplitudes [B,H,S]
 *   - Stateless and thread-safe; calls on one stream run in order.
 */
#ifndef MXFA_H
#define MXFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXFA_OK = 0,
  MXFA_ERR_NULL = 1,        /* a required pointer is NULL */
  MXFA_ERR_SHAPE = 2,       /* B, S or H out of range, S % 32 != 0, Hq % Hkv != 0, bad view */
  MXFA_ERR_UNSUPPORTED = 3, /* D != 128, unknown mode or output dtype, workspace too small */
  MXFA_ERR_ALIGN = 4,       /* pointer not 16-byte aligned or bf16 stride not a multiple of 8 */
  MXFA_ERR_NO_DEVICE = 5,   /* no HIP device, or the current device is not gfx950 */
  MXFA_ERR_HIP = 6          /* the HIP runtime reported an error when launching */
} mxfa_status;

typedef enum { MXFA_QUANT_ROWWISE = 0, MXFA_QUANT_V = 1 } mxfa_quant_mode;
typedef enum { MXFA_OUT_BF16 = 0, MXFA_OUT_F32 = 1 } mxfa_out_dtype;

/* Text of a status code (static storage). */
const char* mxfa_status_string(int status);
/* Detail of the last error returned on this thread ("" if none). */
const char* mxfa_last_error(void);

/* mxfp8_quantize -- MXFP8 encoding of a bf16 [B,S,H,D] tensor.
 * Scale rule: the block's E8M0 exponent k is the smallest integer with amax <= 448 * 2^k (no element
 * saturates; an all-zero block gets byte 0); elements are E4M3 (OCP E4M3FN) codes of x * 2^-k,
 * rounded to nearest even with the sign of zero kept.
 *   mode ROWWISE (Q and K; blocks of 32 along D -- "rowwise MXFP8 bytes", TE #3865 Description):
 *     codes [B,H,S,D], scales [B,H,S,D/32]; tn_codes and tn_amps must be NULL.
 *   mode V (blocks of 32 consecutive tokens per column -- TE #3865 Description, first paragraph;
 *     and the token-normalised copy, one power-of-two amplitude per token over all D -- second
 *     bullet): codes [B,H,D,S], scales [B,H,S/32,D], tn_codes [B,H,S,D], tn_amps [B,H,S].
 *     Either pair may be NULL to skip that output (not both). */
int mxfa_mxfp8_quantize(const void* x_bf16, int B, int S, int H, int D, int64_t sb, int64_t ss, int64_t sh,
                        int mode, uint8_t* codes, uint8_t* scales, uint8_t* tn_codes, uint8_t* tn_amps,
                        void* stream);

/* mxfp8_quantize_kv -- the K and V encodings of one attention call in one launch: K as mode ROWWISE
 * and V as mode V with both outputs, the same bytes as those two mxfp8_quantize calls (TE #3865
 * Description: rowwise K; columnwise V blocks over 32 tokens plus the token-normalised copy). K and V
 * are [B,S,H,D] bf16 views with their own strides; S % 32 == 0; every output is required:
 * k_codes [B,H,S,D], k_scales [B,H,S,D/32], v_codes [B,H,D,S], v_scales [B,H,S/32,D],
 * v_tn_codes [B,H,S,D], v_tn_amps [B,H,S]. One dispatch instead of two; attn_fwd runs it. */
int mxfa_mxfp8_quantize_kv(const void* k_bf16, int64_t ksb, int64_t kss, int64_t ksh, const void* v_bf16,
                           int64_t vsb, int64_t vss, int64_t vsh, int B, int S, int H, int D, uint8_t* k_codes,
                           uint8_t* k_scales, uint8_t* v_codes, uint8_t* v_scales, uint8_t* v_tn_codes,
                           uint8_t* v_tn_amps, void* stream);

/* attn_fwd_completed_blocks -- the completed-block partial (TE #3865 Description, first bullet):
 * for every (b, hq, i), keys j < 32*floor(i/32). Scores t = softmax_scale*log2(e)*(Q^_i . K^_j) come
 * from block-scaled FP8 products; p = 2^(t - T) with an integer running exponent T; P is quantised
 * to E4M3 with one E8M0 scale per (query, 32-key block) and multiplied with the columnwise V.
 * Outputs: o_c fp32 [B,Hq,S,D] = (sum_j p^_j V^_j) / sum_j p_j, lse_c fp32 [B,Hq,S] = natural-log
 * log-sum-exp of the scaled scores. Rows i < 32 have no completed key: o_c = 0, lse_c = -inf. */
int mxfa_attn_fwd_completed_blocks(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                                   const uint8_t* vc, const uint8_t* vcs, int B, int S, int Hq, int Hkv, int D,
                                   float softmax_scale, float* o_c, float* lse_c, void* stream);

/* attn_fwd_own_block -- the own-block partial (TE #3865 Description, second bullet): for every
 * (b, hq, i), keys 32*floor(i/32) <= j <= i, softmax in fp32 of softmax_scale * (Q^_i . K^_j) on the
 * decoded rowwise Q/K, times the decoded token-normalised V. Outputs o_o fp32 [B,Hq,S,D] and
 * lse_o fp32 [B,Hq,S] (natural log). */
int mxfa_attn_fwd_own_block(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                            const uint8_t* vt, const uint8_t* vta, int B, int S, int Hq, int Hkv, int D,
                            float softmax_scale, float* o_o, float* lse_o, void* stream);

/* lse_merge -- merge of the two partials through their log-sum-exps (TE #3865 Description, second
 * bullet): M = max(lse_c, lse_o), w = e^(lse - M), O = (w_c O_c + w_o O_o) / (w_c + w_o),
 * lse = M + ln(w_c + w_o). Partials are fp32 [B,H,S,D] / [B,H,S]. The output is written through the
 * strided view (osb, oss, osh) of a logical [B,S,H,D] tensor as bf16 (round to nearest even) or fp32
 * per out_dtype; lse_out fp32 [B,H,S] may be NULL. */
int mxfa_lse_merge(const float* o_c, const float* lse_c, const float* o_o, const float* lse_o, int B, int S, int H,
                   int D, void* out, int64_t osb, int64_t oss, int64_t osh, int out_dtype, float* lse_out,
                   void* stream);

/* attn_fwd_fused -- both partials and their merge in one kernel (TE #3865 Description, both
 * bullets): per row, the completed blocks as in attn_fwd_completed_blocks, then the row's own block
 * on the token-normalised V (scores on the same block-scaled FP8 product, softmax and P.V in fp32,
 * P not quantised), merged through the log-sum-exps in registers; nothing but the final output and
 * LSE is written. Inputs: the rowwise Q/K codes, the columnwise V codes and the token-normalised V
 * codes in the layouts above. out is a [B,S,Hq,D] view (strides osb, oss, osh) written as bf16
 * (round to nearest even) or fp32 per out_dtype; lse_out fp32 [B,Hq,S] may be NULL. */
int mxfa_attn_fwd_fused(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                        const uint8_t* vc, const uint8_t* vcs, const uint8_t* vt, const uint8_t* vta, int B, int S,
                        int Hq, int Hkv, int D, float softmax_scale, void* out, int64_t osb, int64_t oss,
                        int64_t osh, int out_dtype, float* lse_out, void* stream);

/* attn_fwd_fused_mxfp8 -- attn_fwd_fused with the output itself in MXFP8, for a downstream MXFP8
 * GEMM (the block-scaled O epilogue of cudnn-frontend PR #1088, PR summary: E4M3 O with one UE8M0
 * scale per 32 elements of D, the scales in a separate output). Each row's fp32 output, before any
 * rounding to bf16, is quantised per 32 columns by the rule of mxfa_mxfp8_quantize (smallest k with
 * amax <= 448 * 2^k; codes of x * 2^-k, round to nearest even). o_codes: u8 E4M3 codes through the
 * [B,S,Hq,D] view (element strides osb, oss, osh, multiples of 16; 16-byte aligned); sf_o: u8 E8M0
 * bytes [B,Hq,S,D/32], row-major (this library's own layout, 2^(byte-127)); lse_out fp32 [B,Hq,S]
 * may be NULL. */
int mxfa_attn_fwd_fused_mxfp8(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                              const uint8_t* vc, const uint8_t* vcs, const uint8_t* vt, const uint8_t* vta, int B,
                              int S, int Hq, int Hkv, int D, float softmax_scale, uint8_t* o_codes, int64_t osb,
                              int64_t oss, int64_t osh, uint8_t* sf_o, float* lse_out, void* stream);

/* attn_fwd_leaky -- ordinary causal MXFP8 attention, the variant the method replaces (TE #3865,
 * Description, first paragraph, and the "MXFP8" column under Performance): for every (b, hq, i) all
 * keys j <= i run through the completed-block computation of attn_fwd_completed_blocks, the query's
 * own 32-key block included, with its columnwise V scale (which also covers the block's later
 * tokens: the leak) and its P block's E8M0 taken from the visible keys. For comparison and leak
 * demonstration only. Inputs as attn_fwd_completed_blocks; out is a [B,S,Hq,D] view (strides osb,
 * oss, osh) written as bf16 (round to nearest even) or fp32 per out_dtype; lse_out fp32 [B,Hq,S]
 * (natural log) may be NULL. */
int mxfa_attn_fwd_leaky(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                        const uint8_t* vc, const uint8_t* vcs, int B, int S, int Hq, int Hkv, int D,
                        float softmax_scale, void* out, int64_t osb, int64_t oss, int64_t osh, int out_dtype,
                        float* lse_out, void* stream);

/* Bytes of workspace mxfa_attn_fwd needs (the K and V MXFP8 codes and scales, 256-byte aligned parts). */
size_t mxfa_attn_fwd_workspace_bytes(int B, int S, int Hq, int Hkv, int D);

/* attn_fwd_fused_bf16q -- attn_fwd_fused with Q given as its bf16 [B,S,Hq,D] view (strides qsb, qss,
 * qsh, multiples of 8 elements) instead of its codes: each row of Q is quantised inside the attention
 * kernel by the rule of mxfp8_quantize's rowwise mode (TE #3865 Description: Q in MXFP8 with one E8M0
 * per 32 elements of D), giving the same codes and scales, so the output equals mxfp8_quantize
 * followed by attn_fwd_fused bit for bit. This saves the separate pass over Q. Other arguments as
 * attn_fwd_fused. */
int mxfa_attn_fwd_fused_bf16q(const void* q, int64_t qsb, int64_t qss, int64_t qsh, const uint8_t* kc,
                              const uint8_t* ks, const uint8_t* vc, const uint8_t* vcs, const uint8_t* vt,
                              const uint8_t* vta, int B, int S, int Hq, int Hkv, int D, float softmax_scale,
                              void* out, int64_t osb, int64_t oss, int64_t osh, int out_dtype, float* lse_out,
                              void* stream);

/* attn_fwd -- the whole forward: the K and V quantisations, then attn_fwd_fused_bf16q (which
 * quantises Q in-kernel), in that order on `stream`, using `workspace` (at least
 * mxfa_attn_fwd_workspace_bytes, 256-byte aligned) for the K and V codes. q [B,S,Hq,D], k and v
 * [B,S,Hkv,D] bf16 views; out is a [B,S,Hq,D] view. The result equals the separate calls
 * (mxfp8_quantize of Q, K and V, then attn_fwd_fused) bit for bit. */
int mxfa_attn_fwd(const void* q, int64_t qsb, int64_t qss, int64_t qsh, const void* k, int64_t ksb, int64_t kss,
                  int64_t ksh, const void* v, int64_t vsb, int64_t vss, int64_t vsh, int B, int S, int Hq, int Hkv,
                  int D, float softmax_scale, void* workspace, size_t workspace_bytes, void* out, int64_t osb,
                  int64_t oss, int64_t osh, int out_dtype, float* lse_out, void* stream);

/* attn_fwd_noalloc -- attn_fwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels and result (bit for
 * bit), with the K and V encodings in a static device workspace of the library instead of a
 * caller-provided one. The call itself allocates nothing; the caller still passes q, k, v, out and
 * lse_out. The workspace is a file-scope device array of MXFA_NOALLOC_WORKSPACE_BYTES (256 MiB) held
 * on every device the library runs on until the process ends; its address is looked up on the first
 * call on each device (when the HIP runtime backs the array; later calls touch no allocator). A
 * problem needing more (mxfa_attn_fwd_workspace_bytes above it)
 * is refused with MXFA_ERR_UNSUPPORTED before anything is enqueued. Every call on one device uses the
 * same array, which keeps the last call's contents: calls that overlap on one device (different
 * streams or threads without ordering between them) race and give undefined results. Arguments as
 * attn_fwd, without the workspace. */
#define MXFA_NOALLOC_WORKSPACE_BYTES ((size_t)256 << 20)
int mxfa_attn_fwd_noalloc(const void* q, int64_t qsb, int64_t qss, int64_t qsh, const void* k, int64_t ksb,
                          int64_t kss, int64_t ksh, const void* v, int64_t vsb, int64_t vss, int64_t vsh, int B, int S,
                          int Hq, int Hkv, int D, float softmax_scale, void* out, int64_t osb, int64_t oss,
                          int64_t osh, int out_dtype, float* lse_out, void* stream);

/* Bytes of workspace mxfa_attn_bwd needs (decoded operands: 5 bf16 copies of [B,Hq,S,D] and 3 of
 * [B,Hkv,S,D], plus two [B,Hq,S] fp32 arrays; 256-byte aligned parts). */
size_t mxfa_attn_bwd_workspace_bytes(int B, int S, int Hq, int Hkv, int D);

/* attn_bwd -- backward on decoded operands (TE #3865, Description, backward bullet: BF16 backward on
 * Q/K decoded from their rowwise MXFP8 bytes and V decoded from the token-normalised copy, so no
 * gradient depends on a later token through a shared scale). The gradients of causal softmax
 * attention at those operands, with the forward's O and lse as the softmax statistics:
 *   Delta_i = dO_i . O_i,  P_ij = exp(softmax_scale Q_i . K_j - lse_i) (j <= i),
 *   dS_ij = P_ij (dO_i . V_j - Delta_i),  dQ_i = softmax_scale sum_j dS_ij K_j,
 *   dK_j = softmax_scale sum_i dS_ij Q_i,  dV_j = sum_i P_ij dO_i  (dK, dV summed over the query heads
 *   of a KV head),
 * computed with bf16 operands (P and dS rounded to bf16 before their products) and fp32 accumulation.
 * Inputs: the rowwise Q/K codes and the token-normalised V codes (layouts above); o and dout bf16
 * [B,S,Hq,D] views and dq the bf16 output, all three with the strides (qsb, qss, qsh); dk and dv bf16
 * [B,S,Hkv,D] outputs with the strides (ksb, kss, ksh); lse fp32 [B,Hq,S] (natural log, as the forward
 * writes it). workspace: at least mxfa_attn_bwd_workspace_bytes, 256-byte aligned. */
int mxfa_attn_bwd(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks, const uint8_t* vt,
                  const uint8_t* vta, const void* o, const float* lse, const void* dout, int B, int S, int Hq, int Hkv,
                  int D, float softmax_scale, int64_t qsb, int64_t qss, int64_t qsh, int64_t ksb, int64_t kss,
                  int64_t ksh, void* workspace, size_t workspace_bytes, void* dq, void* dk, void* dv, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MXFA_H */
