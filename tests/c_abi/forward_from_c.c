/*
 * forward_from_c.c -- a plain C consumer of libmxfa (include/mxfa.h), with no Python in the loop.
 *
 * For seeded N(0,1) bf16 inputs (B=1, 2 query heads, 1 KV head, D=128) it
 *   1. encodes Q, K (rowwise) and V (columnwise + token-normalised) with mxfa_mxfp8_quantize, and K
 *      and V again in one launch with mxfa_mxfp8_quantize_kv, and checks every code and scale byte
 *      against the oracle's encoders (TransformerEngine PR #3865, "Description": rowwise Q/K,
 *      columnwise V over 32 tokens, one amplitude per token);
 *   2. runs the whole forward, mxfa_attn_fwd, and checks it equals the chain of separate entry points
 *      (the three quantisations, then mxfa_attn_fwd_fused) bit for bit, as the header promises;
 *   3. at S = 32, where every query has only its own block (no quantised P), checks the own-block
 *      partial entry point against the oracle's within 1e-4 * RMS (LSE within 1e-4; its scores are
 *      exact), and the whole forward against the oracle's merged output within 2e-2 * RMS (its
 *      own-block scores come from the block-scaled FP8 product, whose sums are not exact).
 * Test infrastructure: it links the oracle library, which no product code does.
 * Prints "ALL OK" and exits 0 when every check passes.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mxfa.h"
#include "oracle.h"

static uint64_t rng_state;
static double urand(void) { /* xorshift64*, 53-bit uniform in (0, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return ((double)((rng_state * 0x2545F4914F6CDD1DULL) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}
static double nrand(void) { return sqrt(-2.0 * log(urand())) * cos(6.283185307179586 * urand()); }
static uint16_t to_bf16(float f) { /* round to nearest even (finite inputs) */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

static int failures = 0;
#define HIP_OK(x)                                                                      \
  do {                                                                                 \
    hipError_t e_ = (x);                                                               \
    if (e_ != hipSuccess) {                                                            \
      printf("HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__);                  \
      exit(2);                                                                         \
    }                                                                                  \
  } while (0)
#define MX_OK(x)                                                                       \
  do {                                                                                 \
    int s_ = (x);                                                                      \
    if (s_ != MXFA_OK) {                                                               \
      printf("mxfa status %d (%s) at line %d\n", s_, mxfa_last_error(), __LINE__);     \
      exit(3);                                                                         \
    }                                                                                  \
  } while (0)

static void* dev_alloc(size_t n) {
  void* p = NULL;
  HIP_OK(hipMalloc(&p, n ? n : 1));
  return p;
}
static void* dev_copy(const void* h, size_t n) {
  void* p = dev_alloc(n);
  HIP_OK(hipMemcpy(p, h, n, hipMemcpyHostToDevice));
  return p;
}
static void* host_copy(const void* d, size_t n) {
  void* h = malloc(n ? n : 1);
  HIP_OK(hipMemcpy(h, d, n, hipMemcpyDeviceToHost));
  return h;
}
static void expect_equal(const char* what, const void* a, const void* b, size_t n, int S) {
  const int same = memcmp(a, b, n) == 0;
  printf("S=%d %-44s %s\n", S, what, same ? "identical" : "DIFFER");
  failures += !same;
}

static void run_case(int S) {
  const int B = 1, Hq = 2, Hkv = 1, D = 128;
  const float scale = 1.0f / sqrtf((float)D);
  const size_t nq = (size_t)B * S * Hq * D, nk = (size_t)B * S * Hkv * D;
  uint16_t *q = malloc(nq * 2), *k = malloc(nk * 2), *v = malloc(nk * 2);
  rng_state = 0x9E3779B97F4A7C15ULL ^ (uint64_t)S;
  for (size_t i = 0; i < nq; ++i) q[i] = to_bf16((float)nrand());
  for (size_t i = 0; i < nk; ++i) k[i] = to_bf16((float)nrand());
  for (size_t i = 0; i < nk; ++i) v[i] = to_bf16((float)nrand());
  /* BSHD element strides */
  const int64_t qsb = (int64_t)S * Hq * D, qss = (int64_t)Hq * D, qsh = D;
  const int64_t ksb = (int64_t)S * Hkv * D, kss = (int64_t)Hkv * D, ksh = D;
  void *dq = dev_copy(q, nq * 2), *dk = dev_copy(k, nk * 2), *dv = dev_copy(v, nk * 2);

  /* 1. the encoders against the oracle's */
  const size_t qsn = nq / 32, ksn = nk / 32;
  void *dqc = dev_alloc(nq), *dqs = dev_alloc(qsn), *dkc = dev_alloc(nk), *dks = dev_alloc(ksn);
  void *dvc = dev_alloc(nk), *dvcs = dev_alloc(ksn), *dvt = dev_alloc(nk), *dvta = dev_alloc((size_t)B * Hkv * S);
  MX_OK(mxfa_mxfp8_quantize(dq, B, S, Hq, D, qsb, qss, qsh, MXFA_QUANT_ROWWISE, dqc, dqs, NULL, NULL, NULL));
  MX_OK(mxfa_mxfp8_quantize(dk, B, S, Hkv, D, ksb, kss, ksh, MXFA_QUANT_ROWWISE, dkc, dks, NULL, NULL, NULL));
  MX_OK(mxfa_mxfp8_quantize(dv, B, S, Hkv, D, ksb, kss, ksh, MXFA_QUANT_V, dvc, dvcs, dvt, dvta, NULL));
  HIP_OK(hipDeviceSynchronize());
  uint8_t *oqc = malloc(nq), *oqs = malloc(qsn), *okc = malloc(nk), *oks = malloc(ksn);
  uint8_t *ovc = malloc(nk), *ovcs = malloc(ksn), *ovt = malloc(nk), *ovta = malloc((size_t)B * Hkv * S);
  orc_quantize_rowwise(q, B, S, Hq, D, qsb, qss, qsh, oqc, oqs);
  orc_quantize_rowwise(k, B, S, Hkv, D, ksb, kss, ksh, okc, oks);
  orc_quantize_v(v, B, S, Hkv, D, ksb, kss, ksh, ovc, ovcs, ovt, ovta);
  struct { const char* name; void* dev; uint8_t* ref; size_t n; } enc[] = {
      {"Q rowwise codes", dqc, oqc, nq}, {"Q rowwise scales", dqs, oqs, qsn},
      {"K rowwise codes", dkc, okc, nk}, {"K rowwise scales", dks, oks, ksn},
      {"V columnwise codes", dvc, ovc, nk}, {"V columnwise scales", dvcs, ovcs, ksn},
      {"V token-normalised codes", dvt, ovt, nk}, {"V token amplitudes", dvta, ovta, (size_t)B * Hkv * S}};
  for (size_t i = 0; i < sizeof(enc) / sizeof(enc[0]); ++i) {
    void* h = host_copy(enc[i].dev, enc[i].n);
    expect_equal(enc[i].name, h, enc[i].ref, enc[i].n, S);
    free(h);
  }
  /* ... and K and V in one launch (what mxfa_attn_fwd runs): the same bytes */
  {
    void *ekc = dev_alloc(nk), *eks = dev_alloc(ksn), *evc = dev_alloc(nk), *evcs = dev_alloc(ksn);
    void *evt = dev_alloc(nk), *evta = dev_alloc((size_t)B * Hkv * S);
    MX_OK(mxfa_mxfp8_quantize_kv(dk, ksb, kss, ksh, dv, ksb, kss, ksh, B, S, Hkv, D, ekc, eks, evc, evcs, evt, evta,
                                 NULL));
    HIP_OK(hipDeviceSynchronize());
    struct { const char* name; void* dev; uint8_t* ref; size_t n; } kv[] = {
        {"quantize_kv: K codes", ekc, okc, nk}, {"quantize_kv: K scales", eks, oks, ksn},
        {"quantize_kv: V columnwise codes", evc, ovc, nk}, {"quantize_kv: V columnwise scales", evcs, ovcs, ksn},
        {"quantize_kv: V token-normalised codes", evt, ovt, nk},
        {"quantize_kv: V token amplitudes", evta, ovta, (size_t)B * Hkv * S}};
    for (size_t i = 0; i < sizeof(kv) / sizeof(kv[0]); ++i) {
      void* h = host_copy(kv[i].dev, kv[i].n);
      expect_equal(kv[i].name, h, kv[i].ref, kv[i].n, S);
      free(h);
      HIP_OK(hipFree(kv[i].dev));
    }
  }

  /* 2. the whole forward against the chain of separate calls */
  const size_t ws_bytes = mxfa_attn_fwd_workspace_bytes(B, S, Hq, Hkv, D);
  void* ws = dev_alloc(ws_bytes);
  float *dout = dev_alloc(nq * 4), *dlse = dev_alloc((size_t)B * Hq * S * 4);
  float *dout2 = dev_alloc(nq * 4), *dlse2 = dev_alloc((size_t)B * Hq * S * 4);
  MX_OK(mxfa_attn_fwd(dq, qsb, qss, qsh, dk, ksb, kss, ksh, dv, ksb, kss, ksh, B, S, Hq, Hkv, D, scale, ws, ws_bytes,
                      dout, qsb, qss, qsh, MXFA_OUT_F32, dlse, NULL));
  MX_OK(mxfa_attn_fwd_fused(dqc, dqs, dkc, dks, dvc, dvcs, dvt, dvta, B, S, Hq, Hkv, D, scale, dout2, qsb, qss, qsh,
                            MXFA_OUT_F32, dlse2, NULL));
  HIP_OK(hipDeviceSynchronize());
  float *out = host_copy(dout, nq * 4), *lse = host_copy(dlse, (size_t)B * Hq * S * 4);
  float *out2 = host_copy(dout2, nq * 4), *lse2 = host_copy(dlse2, (size_t)B * Hq * S * 4);
  expect_equal("attn_fwd output = quantise + attn_fwd_fused", out, out2, nq * 4, S);
  expect_equal("attn_fwd LSE = quantise + attn_fwd_fused", lse, lse2, (size_t)B * Hq * S * 4, S);

  /* 3. own block only (S = 32): the own-block partial entry point against the oracle's (exact scores:
   *    1e-4 * RMS, LSE within 1e-4), and the whole forward, whose own-block scores come from the
   *    block-scaled FP8 product, within the forward's 2e-2 * RMS */
  if (S == 32) {
    const size_t nrow = (size_t)B * Hq * S;
    double *oc = malloc(nq * 8), *lc = malloc(nrow * 8), *oo = malloc(nq * 8), *lo = malloc(nrow * 8);
    double *om = malloc(nq * 8), *lm = malloc(nrow * 8);
    orc_attn_completed(oqc, oqs, okc, oks, ovc, ovcs, B, S, Hq, Hkv, D, scale, NULL, S, 0, oc, lc, 0.0, NULL, NULL,
                       NULL, NULL, 0.0, 0);
    orc_attn_own(oqc, oqs, okc, oks, ovt, ovta, B, S, Hq, Hkv, D, scale, NULL, S, oo, lo, 0.0, NULL, NULL, 0.0, 0);
    orc_lse_merge(oc, lc, oo, lo, (int64_t)nrow, D, om, lm);
    float *doo = dev_alloc(nq * 4), *dlo = dev_alloc(nrow * 4);
    MX_OK(mxfa_attn_fwd_own_block(dqc, dqs, dkc, dks, dvt, dvta, B, S, Hq, Hkv, D, scale, doo, dlo, NULL));
    HIP_OK(hipDeviceSynchronize());
    float *go = host_copy(doo, nq * 4), *gl = host_copy(dlo, nrow * 4);
    /* oracle rows and the own-block output are [B,Hq,S,D]; the forward's output is the BSHD view */
    double ss = 0.0, e_own = 0.0, l_own = 0.0, e_fwd = 0.0, l_fwd = 0.0;
    for (int h = 0; h < Hq; ++h)
      for (int s = 0; s < S; ++s) {
        const size_t r = (size_t)h * S + s;
        for (int d = 0; d < D; ++d) {
          ss += om[r * D + d] * om[r * D + d];
          e_own = fmax(e_own, fabs((double)go[r * D + d] - oo[r * D + d]));
          e_fwd = fmax(e_fwd, fabs((double)out[(size_t)s * qss + (size_t)h * qsh + d] - om[r * D + d]));
        }
        l_own = fmax(l_own, fabs((double)gl[r] - lo[r]));
        l_fwd = fmax(l_fwd, fabs((double)lse[(size_t)h * S + s] - lm[r]));
      }
    const double rms = sqrt(ss / (double)nq);
    const int ok_own = e_own <= 1e-4 * rms && l_own <= 1e-4, ok_fwd = e_fwd <= 2e-2 * rms;
    printf("S=%d own-block entry point vs oracle: max|err|/RMS %.3e, max|dlse| %.3e %s\n", S, e_own / rms, l_own,
           ok_own ? "ok" : "FAIL");
    printf("S=%d whole forward vs oracle: max|err|/RMS %.3e, max|dlse| %.3e %s\n", S, e_fwd / rms, l_fwd,
           ok_fwd ? "ok" : "FAIL");
    failures += !ok_own + !ok_fwd;
    free(go); free(gl);
    HIP_OK(hipFree(doo));
    HIP_OK(hipFree(dlo));
    free(oc); free(lc); free(oo); free(lo); free(om); free(lm);
  }
  free(out); free(lse); free(out2); free(lse2);
  free(q); free(k); free(v);
  free(oqc); free(oqs); free(okc); free(oks); free(ovc); free(ovcs); free(ovt); free(ovta);
  void* dev[] = {dq, dk, dv, dqc, dqs, dkc, dks, dvc, dvcs, dvt, dvta, ws, dout, dlse, dout2, dlse2};
  for (size_t i = 0; i < sizeof(dev) / sizeof(dev[0]); ++i) HIP_OK(hipFree(dev[i]));
}

int main(void) {
  setvbuf(stdout, NULL, _IONBF, 0);
  run_case(32);
  run_case(96);
  if (failures) {
    printf("%d check(s) failed\n", failures);
    return 1;
  }
  printf("ALL OK\n");
  return 0;
}
