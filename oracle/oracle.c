/*
 * oracle.c -- plain fp64 CPU oracle for leak-free causal MXFP8 attention.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): used by the tests, the smoke check
 * and the benchmark's CPU-baseline leg, never by the product path.
 *
 * Everything here is written for a reader checking it against the pages by
 * eye: fp64 arithmetic, no blocking, no SIMD, OpenMP only across output rows.
 * Citations name the page and its section:
 *   [TE#3865 Description]  TransformerEngine PR #3865, section "Description"
 *   [TE#3865 commit]       the same PR's own commit message
 *   [cuDNN-FE#1088 summary] cudnn-frontend PR #1088, the PR summary
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   R1  E8M0 rule: the smallest power of two 2^k with amax <= 448 * 2^k, so no
 *       element saturates; an all-zero block gets k = -127 (byte 0).
 *   R2  Element rounding: OCP E4M3FN grid (max 448), round to nearest, ties to
 *       even, saturating, sign of zero kept (negative -> 0x80).
 *   R5  "one power-of-two amplitude per token": one E8M0 per (b, s, kv-head)
 *       over all D, rule R1, and the normalised copy stored as E4M3 codes.
 *   R6  P of the completed blocks is quantised with one E8M0 per (query row,
 *       32-key block aligned to multiples of 32) on p = 2^(t - T), T an integer
 *       upper bound of the row's max of t = scale*log2(e)*q.k; the normaliser l
 *       sums the unquantised p. The code of p is decided on p rounded to fp32:
 *       the PR's tests check the MXFP8 path against an FP32 attention
 *       reference [TE#3865 commits], so P exists as an fp32 tensor before it
 *       is quantised.
 *   R7  Own block: s = scale * q.k on decoded MXFP8 Q/K, p = e^(s - max s) in
 *       full precision (not quantised), V from the token-normalised copy.
 *   R8  A row with no completed key (i < 32) has O_c = 0, lse_c = -inf.
 *   R9  GQA: q-head hq reads kv-head floor(hq / (Hq / Hkv)).
 *   R15 Several valid results: a kernel forms the scores t from a hardware
 *       block-scaled FP8 dot product whose accumulation is not exact (the
 *       gfx950 MFMA cuts small products within groups of 8; measured model and
 *       bound in "the hardware dot product" below), and P.V with the same
 *       instruction. With `allowance` the completed partial also returns, per
 *       output element, the largest change those errors and fp32 evaluation
 *       can make: (i) a P value within its error bound of an E4M3 rounding
 *       midpoint, or a block maximum within it of an E8M0 step, has two valid
 *       codes; (ii) the unquantised p in the normaliser l moves by its bound;
 *       (iii) each 64-key step of P.V may be off by its cut error and one
 *       fp32 unit of the running sum.
 */
#include "oracle.h"

#include <assert.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#define LN2 0.69314718055994530942
#define LOG2E 1.44269504088896340736

/* ---------------------------------------------------------------- codec --- */

/* O1 -- E8M0 exponent [cuDNN-FE#1088 summary: "one UE8M0 scale per 32"],
   rule R1: amax = f * 2^E with f in [1, 2); k = E - 8 when f <= 1.75, else
   E - 7, which is the least k with amax <= 448 * 2^k = 1.75 * 2^(k+8). */
int orc_e8m0_exponent(double amax) {
  assert(amax >= 0.0 && isfinite(amax));
  if (amax == 0.0) return -127;
  int e2;
  double m = frexp(amax, &e2); /* amax = m * 2^e2, m in [0.5, 1) */
  double f = 2.0 * m;          /* f in [1, 2) */
  int E = e2 - 1;
  int k = E - 8 + (f > 1.75 ? 1 : 0);
  if (k < -127) k = -127;
  if (k > 127) k = 127;
  return k;
}

/* O2 -- E4M3 encode (rule R2). Normal codes are 1.mmm * 2^(e-7), e = 1..15,
   the largest finite one is e = 15, m = 6 (448 = 0x7E); subnormals are
   0.mmm * 2^-6 (step 2^-9). The code's integer order follows its magnitude, so
   a mantissa carry into the exponent is just code + 1. */
uint8_t orc_e4m3_encode(double y) {
  assert(!isnan(y));
  uint8_t sign = signbit(y) ? 0x80 : 0x00;
  double a = fabs(y);
  int code;
  if (a >= 448.0) {
    code = 0x7E;
  } else if (a < 0.015625) { /* below 2^-6: subnormal grid, step 2^-9 */
    code = (int)nearbyint(a * 512.0); /* 0..8; 8 is the smallest normal */
  } else {
    int e2;
    double m = frexp(a, &e2);
    int E = e2 - 1;                         /* a = f * 2^E, f in [1, 2) */
    double frac = (2.0 * m - 1.0) * 8.0;    /* mantissa in units of 2^-3 */
    int mant = (int)nearbyint(frac);        /* ties to even */
    code = ((E + 7) << 3) + mant;           /* mant == 8 carries into e */
    if (code > 0x7E) code = 0x7E;
  }
  return (uint8_t)(sign | code);
}

/* O3 -- E4M3 decode. */
double orc_e4m3_decode(uint8_t c) {
  int e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(8.0 + m, e - 10);
  return (c & 0x80) ? -v : v;
}

static double mx_value(uint8_t code, uint8_t scale_byte) {
  return ldexp(orc_e4m3_decode(code), (int)scale_byte - 127);
}

static double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* One MX block: n values -> scale byte and n codes. */
static uint8_t mx_block(const double* x, int n, uint8_t* codes_out, int64_t code_stride) {
  double amax = 0.0;
  for (int r = 0; r < n; ++r) amax = fmax(amax, fabs(x[r]));
  int k = orc_e8m0_exponent(amax);
  for (int r = 0; r < n; ++r) codes_out[r * code_stride] = orc_e4m3_encode(ldexp(x[r], -k));
  return (uint8_t)(k + 127);
}

/* ----------------------------------------------------------- quantisers --- */

/* O4 -- rowwise along D for Q and K [TE#3865 Description: backward on "Q/K
   decoded from their rowwise MXFP8 bytes"]: block g of row (b,s,h) is
   d in [32g, 32g+32). */
void orc_quantize_rowwise(const uint16_t* x, int B, int S, int H, int D, int64_t sb, int64_t ss, int64_t sh,
                          uint8_t* codes, uint8_t* scales) {
  assert(D % 32 == 0);
  const int G = D / 32;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b)
    for (int s = 0; s < S; ++s)
      for (int h = 0; h < H; ++h) {
        double blk[32];
        const uint16_t* row = x + b * sb + s * ss + h * sh;
        int64_t out_row = (((int64_t)b * H + h) * S + s);
        for (int g = 0; g < G; ++g) {
          for (int r = 0; r < 32; ++r) blk[r] = bf16_value(row[32 * g + r]);
          scales[out_row * G + g] = mx_block(blk, 32, codes + out_row * D + 32 * g, 1);
        }
      }
}

/* MXFP8 of an output [cudnn-frontend PR #1088, PR summary: E4M3 O with one
   UE8M0 scale per 32 elements of D]: the rows of x (fp64 values, n rows of D)
   in blocks of 32 along D by O1 and O2, exactly as O4 does for bf16 rows. */
void orc_quantize_rows_f64(const double* x, int64_t n, int D, uint8_t* codes, uint8_t* scales) {
  assert(D % 32 == 0);
  const int G = D / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r)
    for (int g = 0; g < G; ++g)
      scales[r * G + g] = mx_block(x + r * D + 32 * g, 32, codes + r * D + 32 * g, 1);
}

/* O5 -- V columnwise: block u of column (b,h,d) is tokens [32u, 32u+32)
   [TE#3865 Description: "A columnwise MXFP8 V scale is shared by 32
   consecutive tokens"]. O6 -- the token-normalised copy: one amplitude per
   (b,s,h) over all D [TE#3865 Description: "one power-of-two amplitude per
   token"], reading R5. */
void orc_quantize_v(const uint16_t* v, int B, int S, int H, int D, int64_t sb, int64_t ss, int64_t sh,
                    uint8_t* col_codes, uint8_t* col_scales, uint8_t* tn_codes, uint8_t* tn_amps) {
  assert(S % 32 == 0);
  const int U = S / 32;
  if (col_codes && col_scales) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < H; ++h)
        for (int u = 0; u < U; ++u)
          for (int d = 0; d < D; ++d) {
            double blk[32];
            for (int r = 0; r < 32; ++r) blk[r] = bf16_value(v[b * sb + (int64_t)(32 * u + r) * ss + h * sh + d]);
            int64_t col = ((int64_t)b * H + h) * D + d; /* codes [B,H,D,S] */
            col_scales[(((int64_t)b * H + h) * U + u) * D + d] =
                mx_block(blk, 32, col_codes + col * S + 32 * u, 1);
          }
  }
  if (tn_codes && tn_amps) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < H; ++h)
        for (int s = 0; s < S; ++s) {
          double* row = (double*)malloc(sizeof(double) * D);
          for (int d = 0; d < D; ++d) row[d] = bf16_value(v[b * sb + (int64_t)s * ss + h * sh + d]);
          int64_t r = ((int64_t)b * H + h) * S + s;
          tn_amps[r] = mx_block(row, D, tn_codes + r * D, 1);
          free(row);
        }
  }
}

/* ------------------------------------------------------ decoded operands --- */

/* Decoded operand tensors, all token-major [B,H,S,D] in fp64. */
static double* decode_rowwise(const uint8_t* c, const uint8_t* s, int B, int H, int S, int D) {
  int64_t n = (int64_t)B * H * S * D;
  double* out = (double*)malloc(sizeof(double) * n);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = mx_value(c[i], s[i / 32]);
  return out;
}

static double* decode_vcol(const uint8_t* c, const uint8_t* s, int B, int H, int S, int D) {
  const int U = S / 32;
  double* out = (double*)malloc(sizeof(double) * (int64_t)B * H * S * D);
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int t = 0; t < S; ++t)
        for (int d = 0; d < D; ++d) {
          int64_t bh = (int64_t)b * H + h;
          out[(bh * S + t) * D + d] = mx_value(c[(bh * D + d) * S + t], s[(bh * U + t / 32) * D + d]);
        }
  return out;
}

static double* decode_vtn(const uint8_t* c, const uint8_t* a, int B, int H, int S, int D) {
  int64_t n = (int64_t)B * H * S * D;
  double* out = (double*)malloc(sizeof(double) * n);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = mx_value(c[i], a[i / D]);
  return out;
}

static double* bf16_tensor(const uint16_t* x, int64_t sb, int64_t ss, int64_t sh, int B, int S, int H, int D) {
  double* out = (double*)malloc(sizeof(double) * (int64_t)B * H * S * D);
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int s = 0; s < S; ++s)
        for (int d = 0; d < D; ++d)
          out[((((int64_t)b * H + h) * S) + s) * D + d] = bf16_value(x[b * sb + s * ss + h * sh + d]);
  return out;
}

static double dot(const double* a, const double* b, int D) {
  double acc = 0.0;
  for (int d = 0; d < D; ++d) acc += a[d] * b[d];
  return acc;
}

/* MX quantise-dequantise of one block of P (reading R6): the code is decided on
   each p rounded to fp32, and the block scale on the fp32 maximum. Returns the
   block exponent k; codes (may be NULL) receives the n codes. */
static int quantize_p_block(const double* p, double* phat, uint8_t* codes, int n) {
  double amax = 0.0;
  for (int r = 0; r < n; ++r) amax = fmax(amax, (double)(float)p[r]);
  int k = orc_e8m0_exponent(amax);
  for (int r = 0; r < n; ++r) {
    uint8_t c = orc_e4m3_encode(ldexp((double)(float)p[r], -k));
    if (codes) codes[r] = c;
    phat[r] = ldexp(orc_e4m3_decode(c), k);
  }
  return k;
}

/* ------------------------------------------- the hardware dot product --- */

/* Reading R15: a kernel forms Q.K^T and P.V with the block-scaled FP8 MFMA of
   gfx950, whose sum is not the exact one. What the probe tests measured, and
   what the bounds below assume:
     - each product of two E4M3 values (times their two scales) is exact;
     - within each group of 8 consecutive products of one 32-element scale
       block, every product is cut toward zero to a multiple of 2^(E - 13),
       where E is the group's largest exponent sum e(a) + e(b) plus the two
       scale exponents, e(code) being the code's exponent field minus 7 (a
       zero field, zero or subnormal, is counted as -6, the largest value the
       hardware could give it);
     - the cut products of a 64-product step are summed and rounded to fp32,
       and each step's result is added to the fp32 accumulator with one more
       rounding (within one fp32 unit in the last place each).
   The bound of one step is the sum over its products of |p - cut(p)|. */
static int mfma_exp(uint8_t code) {
  int e = (code >> 3) & 15;
  return e == 0 ? -6 : e - 7;
}

/* Value (O3) and MFMA exponent of each code, tabulated once (the bounds
   evaluate them billions of times). */
static double code_value[256];
static int code_exp[256];
static void init_code_tables(void) {
  static int done = 0;
  if (done) return;
  for (int c = 0; c < 256; ++c) {
    code_value[c] = ((c & 0x7F) == 0x7F) ? 0.0 : orc_e4m3_decode((uint8_t)c);
    code_exp[c] = mfma_exp((uint8_t)c);
  }
  done = 1;
}

/* One fp32 unit in the last place at magnitude a >= 0. */
static double ulp32(double a) {
  if (a < ldexp(1.0, -126)) return ldexp(1.0, -149);
  int e;
  frexp(a, &e); /* a in [2^(e-1), 2^e) */
  return ldexp(1.0, e - 1 - 23);
}

/* Cut error of one step of 64 products a[i] * b[i] (E4M3 codes), with scale
   exponents sa[i / 32], sb[i / 32]; *sum receives the exact sum of the
   products and *mag the sum of their magnitudes. */
static double mfma_step_cut(const uint8_t* a, const uint8_t* b, const int* sa, const int* sb, double* sum,
                            double* mag) {
  double cut = 0.0, tot = 0.0, m = 0.0;
  for (int g = 0; g < 8; ++g) {
    const int blk = g / 4, sc = sa[blk] + sb[blk];
    int E = -100000;
    for (int i = 8 * g; i < 8 * g + 8; ++i) {
      int e = code_exp[a[i]] + code_exp[b[i]];
      if (e > E) E = e;
    }
    /* in units of the group's scale 2^sc, the cut is at 2^(E - 13) */
    const double gran = ldexp(1.0, E - 13), scale = ldexp(1.0, sc);
    double gcut = 0.0, gtot = 0.0, gmag = 0.0;
    for (int i = 8 * g; i < 8 * g + 8; ++i) {
      double prod = code_value[a[i]] * code_value[b[i]];
      double kept = floor(fabs(prod) / gran) * gran;
      gcut += fabs(prod) - kept;
      gtot += prod;
      gmag += fabs(prod);
    }
    cut += gcut * scale;
    tot += gtot * scale;
    m += gmag * scale;
  }
  *sum = tot;
  *mag = m;
  return cut;
}

/* Bound of |hardware score - exact q.k| for one query row and one key row
   (128 codes, 4 scale bytes each) on the two 64-wide steps over D. */
static double score_bound(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks) {
  int sq[4], sk[4];
  for (int g = 0; g < 4; ++g) {
    sq[g] = (int)qs[g] - 127;
    sk[g] = (int)ks[g] - 127;
  }
  double s0, s1, m0, m1;
  double c0 = mfma_step_cut(qc, kc, sq, sk, &s0, &m0);
  double c1 = mfma_step_cut(qc + 64, kc + 64, sq + 2, sk + 2, &s1, &m1);
  return c0 + c1 + ulp32(fabs(s0) + c0) + ulp32(fabs(s0 + s1) + c0 + c1);
}

void orc_score_bound(const uint8_t* ac, const uint8_t* as, const uint8_t* bc, const uint8_t* bs, int64_t na,
                     int64_t nb, double* out) {
  init_code_tables();
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < na; ++i)
    for (int64_t j = 0; j < nb; ++j) out[i * nb + j] = score_bound(ac + i * 128, as + i * 4, bc + j * 128, bs + j * 4);
}

/* ------------------------------------------------------- partial kernels --- */

/* Bound of the relative error of a kernel's p for key j (reading R15), in two
   parts, both in log2 units before the factor ln 2:
     - the hardware dot product: hw_err times its bound dot_bound (above),
       scaled by sigma * log2(e);
     - fp32 evaluation: t = sigma log2(e) q.k with an fp32 factor, t - T - k
       (and the block exponent's log2 maximum) rounded in fp32 with a running
       exponent T that lies within the row's largest |t| plus one of zero:
       2^-22 (|t| + tabs + 16) with tabs the row's largest |t|;
   plus 2^-22 for the fp32 exponential itself. */
static double p_rel_bound(double dot_bound, double sigma, double t, double tabs, double hw_err) {
  double dt = sigma * LOG2E * hw_err * dot_bound + ldexp(fabs(t) + tabs + 16.0, -22);
  return LN2 * dt + ldexp(1.0, -22);
}

/* Deterministic jitter in [-1, 1] for (row, key) (splitmix64 of the pair). */
static double jitter_unit(uint64_t seed, int64_t row, int64_t j) {
  uint64_t z = seed ^ ((uint64_t)row * 0x9E3779B97F4A7C15ull) ^ ((uint64_t)j * 0xD1B54A32D192ED03ull);
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) * ldexp(1.0, -52) - 1.0;
}

/* MXFP8 codes of one query row's operands, for the hardware bounds of
   reading R15: the query row's 128 codes and 4 scale bytes, its kv head's K
   codes [S,128] and scales [S,4], and (completed partial only) its V
   columnwise codes [128,S] and scales [S/32,128]. */
typedef struct {
  const uint8_t *qc, *qs, *kc, *ks, *vc, *vcs;
  int S;
} RowCodes;

/* O7 -- completed-block partial of one query row [TE#3865 Description, first
   bullet: keys j < 32 * floor(i / 32)], or, with `leaky`, the ordinary causal
   MXFP8 row over j <= i. Keys [0, n) with n as above; P blocks are the 32-key
   blocks aligned to multiples of 32 (the last one partial when leaky).
   quantize_p = 0 replaces the P quantiser by the identity.
   With `allow` (D values) and the row's codes `rc` it also returns the R15
   allowance of the row for a kernel on the block-scaled FP8 MFMA (hw_err
   times the measured error model; 0 leaves fp32 evaluation only), and with
   `allow_code` (D values, may be NULL) its part (i) alone: the change
   alternative valid P codes can make.
   jitter != 0 moves every score by jitter * (its error bound) * u, u in
   [-1, 1] from (jitter_seed, row, key): a model of a kernel's score error,
   used only to pin the allowance. */
static void completed_row(const double* q, const double* K, const double* V, const RowCodes* rc, int i, int D,
                          double sigma, int quantize_p, int t_shift, int leaky, double hw_err, double jitter,
                          uint64_t jitter_seed, int64_t row_id, double* o, double* lse, double* allow,
                          double* allow_code, double* allow_pv, double* lse_err) {
  int n = leaky ? i + 1 : 32 * (i / 32);
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  if (allow)
    for (int d = 0; d < D; ++d) allow[d] = 0.0;
  if (allow_code)
    for (int d = 0; d < D; ++d) allow_code[d] = 0.0;
  if (allow_pv)
    for (int d = 0; d < D; ++d) allow_pv[d] = 0.0;
  if (lse_err) *lse_err = 0.0;
  if (n == 0) { /* R8 */
    *lse = -INFINITY;
    return;
  }
  /* keys of the 64-key MFMA steps that cover [0, n), within the sequence */
  const int nsteps = (n + 63) / 64, ncover = rc ? (nsteps * 64 < rc->S ? nsteps * 64 : rc->S) : n;
  double* t = (double*)malloc(sizeof(double) * n);
  double* p = (double*)malloc(sizeof(double) * n);
  double* phat = (double*)malloc(sizeof(double) * n);
  double* rel = (double*)malloc(sizeof(double) * n);
  double* alt = (double*)calloc(n, sizeof(double)); /* largest |change| of phat_j over valid codes */
  uint8_t* pcode = (uint8_t*)calloc(nsteps * 64, 1); /* P codes; keys past n hold code 0 */
  int* pk = (int*)malloc(sizeof(int) * nsteps * 2);   /* P block exponents */
  for (int u = 0; u < nsteps * 2; ++u) pk[u] = -127;
  double tmax = -INFINITY, tabs = 0.0;
  for (int j = 0; j < n; ++j) {
    t[j] = sigma * LOG2E * dot(q, K + (int64_t)j * D, D);
    tabs = fmax(tabs, fabs(t[j]));
  }
  for (int j = 0; j < n; ++j) {
    if (allow || jitter != 0.0) {
      double b = rc ? score_bound(rc->qc, rc->qs, rc->kc + (int64_t)j * 128, rc->ks + (int64_t)j * 4) : 0.0;
      rel[j] = p_rel_bound(b, sigma, t[j], tabs, hw_err);
    }
    if (jitter != 0.0) t[j] += jitter * (rel[j] / LN2) * jitter_unit(jitter_seed, row_id, j);
    tmax = fmax(tmax, t[j]);
  }
  double T = ceil(tmax) + t_shift; /* integer exponent offset */
  double l = 0.0;
  for (int j = 0; j < n; ++j) {
    p[j] = exp2(t[j] - T);
    l += p[j];
  }
  for (int u0 = 0; u0 < n; u0 += 32) {
    int m = (n - u0 < 32) ? n - u0 : 32;
    if (!quantize_p) {
      for (int r = 0; r < m; ++r) phat[u0 + r] = p[u0 + r];
      continue;
    }
    pk[u0 / 32] = quantize_p_block(p + u0, phat + u0, pcode + u0, m);
    if (!allow) continue;
    /* R15: element codes within the bound of a midpoint, and block scales
       within the bound of an E8M0 step, each give an alternative value. */
    double amax = 0.0, rmax = 0.0;
    for (int r = 0; r < m; ++r) {
      amax = fmax(amax, (double)(float)p[u0 + r]);
      rmax = fmax(rmax, rel[u0 + r]);
    }
    int klo = orc_e8m0_exponent(amax * (1.0 - rmax)), khi = orc_e8m0_exponent(amax * (1.0 + rmax));
    if (klo == -127) {
      /* a block clamped at the smallest scale: a kernel whose running exponent
         T lies below this row's final one sees it unclamped, so its codes may
         be those of any larger scale (the values, at most 448 * 2^-127, only
         bound the change: each code moves p^ by at most 2p + p^) */
      for (int r = 0; r < m; ++r) alt[u0 + r] = fmax(alt[u0 + r], 2.0 * p[u0 + r] + phat[u0 + r]);
    }
    for (int r = 0; r < m; ++r) {
      double y = (double)(float)p[u0 + r];
      for (int kk = klo; kk <= khi; ++kk) {
        double lo = ldexp(orc_e4m3_decode(orc_e4m3_encode(ldexp(y * (1.0 - rel[u0 + r]), -kk))), kk);
        double hi = ldexp(orc_e4m3_decode(orc_e4m3_encode(ldexp(y * (1.0 + rel[u0 + r]), -kk))), kk);
        double ch = fmax(fabs(lo - phat[u0 + r]), fabs(hi - phat[u0 + r]));
        /* values between lo and hi map to codes between them: lo and hi bound the change */
        alt[u0 + r] = fmax(alt[u0 + r], ch);
      }
    }
  }
  for (int j = 0; j < n; ++j)
    for (int d = 0; d < D; ++d) o[d] += phat[j] * V[(int64_t)j * D + d];
  for (int d = 0; d < D; ++d) o[d] /= l;
  if (allow) {
    /* (i) alternative codes */
    for (int j = 0; j < n; ++j)
      if (alt[j] > 0.0)
        for (int d = 0; d < D; ++d) allow[d] += alt[j] * fabs(V[(int64_t)j * D + d]);
    if (allow_code)
      for (int d = 0; d < D; ++d) allow_code[d] = allow[d] / l;
    /* (iii) P.V on the block-scaled MFMA: per 64-key step and column, the cut
       error of its products and one fp32 unit of the running sum */
    if (rc && quantize_p) {
      const int U = rc->S / 32;
      for (int d = 0; d < D; ++d) {
        double run = 0.0;
        for (int st = 0; st < nsteps; ++st) {
          uint8_t vcode[64];
          int sv[2];
          for (int r = 0; r < 64; ++r) {
            int j = 64 * st + r;
            vcode[r] = j < ncover ? rc->vc[(int64_t)d * rc->S + j] : 0;
          }
          for (int h = 0; h < 2; ++h) {
            int u = 2 * st + h;
            sv[h] = u < U ? (int)rc->vcs[(int64_t)u * D + d] - 127 : -127;
          }
          double sum, mag;
          double cut = mfma_step_cut(pcode + 64 * st, vcode, pk + 2 * st, sv, &sum, &mag);
          run += mag;
          allow[d] += hw_err * (cut + ulp32(run));
          if (allow_pv) allow_pv[d] += hw_err * (cut + ulp32(run)) / l;
        }
      }
    }
    for (int d = 0; d < D; ++d) allow[d] /= l;
    /* (ii) the normaliser: l = sum p moves by at most sum rel_j p_j */
    double dl = 0.0;
    for (int j = 0; j < n; ++j) dl += rel[j] * p[j];
    for (int d = 0; d < D; ++d) allow[d] += fabs(o[d]) * dl / l;
    if (lse_err) *lse_err = dl / l; /* |d lse| <= |dl| / l */
  }
  *lse = LN2 * (T + log2(l));
  free(t);
  free(p);
  free(phat);
  free(rel);
  free(alt);
  free(pcode);
  free(pk);
}

/* O8 -- own-block partial of one query row [TE#3865 Description, second
   bullet], reading R7: keys 32*floor(i/32) .. i, full-precision softmax.
   With `allow` and the row's codes `rc`, also the R15 allowance for a kernel
   whose scores carry the hardware dot-product error (each p_j moves by at
   most its relative bound rel_j, so O_o moves by at most
   sum_j rel_j p_j |V_j - O_o| / l) and the bound of its lse error
   (sum_j rel_j p_j / l). jitter: as for O7. */
static void own_row(const double* q, const double* K, const double* Vt, const RowCodes* rc, int i, int D,
                    double sigma, double hw_err, double jitter, uint64_t jitter_seed, int64_t row_id, double* o,
                    double* lse, double* allow, double* lse_err) {
  int j0 = 32 * (i / 32);
  double s[32], p[32], rel[32];
  double m = -INFINITY, tabs = 0.0;
  for (int j = j0; j <= i; ++j) {
    s[j - j0] = sigma * dot(q, K + (int64_t)j * D, D);
    tabs = fmax(tabs, fabs(s[j - j0] * LOG2E));
  }
  for (int j = j0; j <= i; ++j) {
    if (allow || jitter != 0.0) {
      double b = rc ? score_bound(rc->qc, rc->qs, rc->kc + (int64_t)j * 128, rc->ks + (int64_t)j * 4) : 0.0;
      rel[j - j0] = p_rel_bound(b, sigma, s[j - j0] * LOG2E, tabs, hw_err);
    }
    if (jitter != 0.0) s[j - j0] += jitter * (rel[j - j0] / LN2) / LOG2E * jitter_unit(jitter_seed, row_id, j);
    m = fmax(m, s[j - j0]);
  }
  double l = 0.0;
  for (int j = j0; j <= i; ++j) {
    p[j - j0] = exp(s[j - j0] - m);
    l += p[j - j0];
  }
  for (int d = 0; d < D; ++d) {
    double acc = 0.0;
    for (int j = j0; j <= i; ++j) acc += p[j - j0] * Vt[(int64_t)j * D + d];
    o[d] = acc / l;
  }
  *lse = m + log(l);
  if (allow) {
    double dl = 0.0;
    for (int j = j0; j <= i; ++j) dl += rel[j - j0] * p[j - j0];
    for (int d = 0; d < D; ++d) {
      double a = 0.0;
      for (int j = j0; j <= i; ++j) a += rel[j - j0] * p[j - j0] * fabs(Vt[(int64_t)j * D + d] - o[d]);
      allow[d] = a / l;
    }
    if (lse_err) *lse_err = dl / l;
  }
}

/* O9 -- merge through the log-sum-exps [TE#3865 Description, second bullet:
   "merged with the cuDNN partial through the two log-sum-exps"]. */
static void merge_row(const double* oc, double lc, const double* oo, double lo, int D, double* o, double* lse) {
  double M = fmax(lc, lo);
  double wc = (lc == -INFINITY) ? 0.0 : exp(lc - M);
  double wo = (lo == -INFINITY) ? 0.0 : exp(lo - M);
  for (int d = 0; d < D; ++d) o[d] = (wc * oc[d] + wo * oo[d]) / (wc + wo);
  *lse = M + log(wc + wo);
}

void orc_lse_merge(const double* oc, const double* lsec, const double* oo, const double* lseo, int64_t n, int D,
                   double* o, double* lse) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) merge_row(oc + r * D, lsec[r], oo + r * D, lseo[r], D, o + r * D, lse + r);
}

/* --------------------------------------------------------- row drivers --- */

enum { PART_COMPLETED, PART_LEAKY, PART_OWN, PART_TEXTBOOK };

static int row_index(const int32_t* rows, int r) { return rows ? rows[r] : r; }

/* Runs one partial over every (b, hq, listed row). Q, K, V are decoded
   token-major [B,H,S,D] tensors; qc..vcs (may all be NULL) their MXFP8 codes
   in the library layouts, for the hardware bounds. */
static void run_rows(int part, const double* Q, const double* K, const double* V, const uint8_t* qc,
                     const uint8_t* qs, const uint8_t* kc, const uint8_t* ks, const uint8_t* vc, const uint8_t* vcs,
                     int B, int S, int Hq, int Hkv, int D, float scale, const int32_t* rows, int nrows, int quantize_p,
                     int t_shift, double hw_err, double jitter, uint64_t jitter_seed, double* o, double* lse,
                     double* allow, double* allow_code, double* allow_pv, double* lse_err) {
  assert(Hq % Hkv == 0);
  const int G = Hq / Hkv;
  const double sigma = (double)scale;
  if (!rows) assert(nrows == S);
#pragma omp parallel for collapse(3) schedule(dynamic, 4)
  for (int b = 0; b < B; ++b)
    for (int hq = 0; hq < Hq; ++hq)
      for (int r = 0; r < nrows; ++r) {
        int i = row_index(rows, r);
        assert(i >= 0 && i < S);
        int hk = hq / G; /* R9 */
        const double* q = Q + (((int64_t)b * Hq + hq) * S + i) * D;
        const double* Kh = K + ((int64_t)b * Hkv + hk) * S * D;
        const double* Vh = V + ((int64_t)b * Hkv + hk) * S * D;
        int64_t orow = ((int64_t)b * Hq + hq) * nrows + r;
        RowCodes rcodes, *rc = NULL;
        if (qc && kc) {
          const int64_t bhq = (int64_t)b * Hq + hq, bhk = (int64_t)b * Hkv + hk;
          rcodes.qc = qc + (bhq * S + i) * 128;
          rcodes.qs = qs + (bhq * S + i) * 4;
          rcodes.kc = kc + bhk * S * 128;
          rcodes.ks = ks + bhk * S * 4;
          rcodes.vc = vc ? vc + bhk * 128 * S : NULL;
          rcodes.vcs = vcs ? vcs + bhk * (S / 32) * 128 : NULL;
          rcodes.S = S;
          rc = &rcodes;
        }
        if (part == PART_OWN) {
          own_row(q, Kh, Vh, rc, i, D, sigma, hw_err, jitter, jitter_seed, ((int64_t)b * Hq + hq) * S + i,
                  o + orow * D, lse + orow, allow ? allow + orow * D : NULL, lse_err ? lse_err + orow : NULL);
        } else if (part == PART_TEXTBOOK) {
          double* s = (double*)malloc(sizeof(double) * (i + 1));
          double m = -INFINITY, l = 0.0;
          for (int j = 0; j <= i; ++j) {
            s[j] = sigma * dot(q, Kh + (int64_t)j * D, D);
            m = fmax(m, s[j]);
          }
          for (int d = 0; d < D; ++d) o[orow * D + d] = 0.0;
          for (int j = 0; j <= i; ++j) {
            double p = exp(s[j] - m);
            l += p;
            for (int d = 0; d < D; ++d) o[orow * D + d] += p * Vh[(int64_t)j * D + d];
          }
          for (int d = 0; d < D; ++d) o[orow * D + d] /= l;
          lse[orow] = m + log(l);
          free(s);
        } else {
          completed_row(q, Kh, Vh, rc, i, D, sigma, quantize_p, t_shift, part == PART_LEAKY, hw_err, jitter, jitter_seed,
                        ((int64_t)b * Hq + hq) * S + i, o + orow * D, lse + orow, allow ? allow + orow * D : NULL,
                        allow_code ? allow_code + orow * D : NULL, allow_pv ? allow_pv + orow * D : NULL,
                        lse_err ? lse_err + orow : NULL);
        }
      }
}

void orc_attn_completed(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                        const uint8_t* vc, const uint8_t* vcs, int B, int S, int Hq, int Hkv, int D, float scale,
                        const int32_t* rows, int nrows, int t_shift, double* o, double* lse, double hw_err,
                        double* allowance, double* allowance_code, double* allowance_pv, double* lse_err,
                        double jitter, uint64_t jitter_seed) {
  init_code_tables();
  double* Q = decode_rowwise(qc, qs, B, Hq, S, D);
  double* K = decode_rowwise(kc, ks, B, Hkv, S, D);
  double* V = decode_vcol(vc, vcs, B, Hkv, S, D);
  run_rows(PART_COMPLETED, Q, K, V, qc, qs, kc, ks, vc, vcs, B, S, Hq, Hkv, D, scale, rows, nrows, 1, t_shift,
           hw_err, jitter, jitter_seed, o, lse, allowance, allowance_code, allowance_pv, lse_err);
  free(Q);
  free(K);
  free(V);
}

void orc_attn_leaky(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks, const uint8_t* vc,
                    const uint8_t* vcs, int B, int S, int Hq, int Hkv, int D, float scale, const int32_t* rows,
                    int nrows, double* o, double* lse, double hw_err, double* allowance, double* allowance_code,
                    double* allowance_pv, double* lse_err, double jitter, uint64_t jitter_seed) {
  init_code_tables();
  double* Q = decode_rowwise(qc, qs, B, Hq, S, D);
  double* K = decode_rowwise(kc, ks, B, Hkv, S, D);
  double* V = decode_vcol(vc, vcs, B, Hkv, S, D);
  run_rows(PART_LEAKY, Q, K, V, qc, qs, kc, ks, vc, vcs, B, S, Hq, Hkv, D, scale, rows, nrows, 1, 0, hw_err, jitter,
           jitter_seed, o, lse, allowance, allowance_code, allowance_pv, lse_err);
  free(Q);
  free(K);
  free(V);
}

void orc_attn_own(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks, const uint8_t* vt,
                  const uint8_t* vta, int B, int S, int Hq, int Hkv, int D, float scale, const int32_t* rows,
                  int nrows, double* o, double* lse, double hw_err, double* allowance, double* lse_err,
                  double jitter, uint64_t jitter_seed) {
  init_code_tables();
  double* Q = decode_rowwise(qc, qs, B, Hq, S, D);
  double* K = decode_rowwise(kc, ks, B, Hkv, S, D);
  double* V = decode_vtn(vt, vta, B, Hkv, S, D);
  run_rows(PART_OWN, Q, K, V, qc, qs, kc, ks, NULL, NULL, B, S, Hq, Hkv, D, scale, rows, nrows, 0, 0, hw_err, jitter,
           jitter_seed, o, lse, allowance, NULL, NULL, lse_err);
  free(Q);
  free(K);
  free(V);
}

void orc_attn_reference(const uint16_t* q, int64_t qsb, int64_t qss, int64_t qsh, const uint16_t* k, int64_t ksb,
                        int64_t kss, int64_t ksh, const uint16_t* v, int64_t vsb, int64_t vss, int64_t vsh, int B,
                        int S, int Hq, int Hkv, int D, float scale, const int32_t* rows, int nrows, double* o,
                        double* lse) {
  double* Q = bf16_tensor(q, qsb, qss, qsh, B, S, Hq, D);
  double* K = bf16_tensor(k, ksb, kss, ksh, B, S, Hkv, D);
  double* V = bf16_tensor(v, vsb, vss, vsh, B, S, Hkv, D);
  run_rows(PART_TEXTBOOK, Q, K, V, NULL, NULL, NULL, NULL, NULL, NULL, B, S, Hq, Hkv, D, scale, rows, nrows, 0, 0,
           0.0, 0.0, 0, o, lse, NULL, NULL, NULL, NULL);
  free(Q);
  free(K);
  free(V);
}

void orc_attn_identity(const uint16_t* q, int64_t qsb, int64_t qss, int64_t qsh, const uint16_t* k, int64_t ksb,
                       int64_t kss, int64_t ksh, const uint16_t* v, int64_t vsb, int64_t vss, int64_t vsh, int B,
                       int S, int Hq, int Hkv, int D, float scale, const int32_t* rows, int nrows, double* o,
                       double* lse) {
  double* Q = bf16_tensor(q, qsb, qss, qsh, B, S, Hq, D);
  double* K = bf16_tensor(k, ksb, kss, ksh, B, S, Hkv, D);
  double* V = bf16_tensor(v, vsb, vss, vsh, B, S, Hkv, D);
  int64_t n = (int64_t)B * Hq * nrows;
  double* oc = (double*)malloc(sizeof(double) * n * D);
  double* oo = (double*)malloc(sizeof(double) * n * D);
  double* lc = (double*)malloc(sizeof(double) * n);
  double* lo = (double*)malloc(sizeof(double) * n);
  run_rows(PART_COMPLETED, Q, K, V, NULL, NULL, NULL, NULL, NULL, NULL, B, S, Hq, Hkv, D, scale, rows, nrows, 0, 0,
           0.0, 0.0, 0, oc, lc, NULL, NULL, NULL, NULL);
  run_rows(PART_OWN, Q, K, V, NULL, NULL, NULL, NULL, NULL, NULL, B, S, Hq, Hkv, D, scale, rows, nrows, 0, 0, 0.0,
           0.0, 0, oo, lo, NULL, NULL, NULL, NULL);
  orc_lse_merge(oc, lc, oo, lo, n, D, o, lse);
  free(oc);
  free(oo);
  free(lc);
  free(lo);
  free(Q);
  free(K);
  free(V);
}

/* ------------------------------------------------------------- backward --- */

/* Backward on decoded operands [TE#3865 Description, backward bullet: BF16
   backward on Q/K decoded from their rowwise MXFP8 bytes and V decoded from
   the token-normalised copy]: the gradients of causal softmax attention
   O = softmax(scale Q K^T) V at the real-valued operands Q, K, V, with the
   forward's O and lse (natural log) as the softmax statistics and dO the
   output gradient:
     Delta_i = sum_d dO_i,d O_i,d
     P_ij    = exp(scale Q_i . K_j - lse_i)                    (j <= i)
     dS_ij   = P_ij (dO_i . V_j - Delta_i)
     dQ_i    = scale sum_{j <= i} dS_ij K_j
     dK_j    = scale sum_{hq of kv head} sum_{i >= j} dS_ij Q_i
     dV_j    = sum_{hq of kv head} sum_{i >= j} P_ij dO_i
   Q, O, dO [B,Hq,S,D], K, V [B,Hkv,S,D], lse [B,Hq,S]. dq for the query rows
   qrows (nq of them; NULL: all S) into [B,Hq,nq,D]; dk and dv for the key rows
   krows (nk; NULL: all) into [B,Hkv,nk,D]. Any output may be NULL.
   aq, ak, av (optional, shaped as dq, dk, dv): reading R16, the bf16 backward's
   operand rounding -- P and dS enter their products rounded to bf16 (relative
   error at most 2^-8, bf16's unit roundoff) -- bounded per element: aq = 2^-8
   scale sum_j |dS_ij| |K_j|, ak = 2^-8 scale sum_i |dS_ij| |Q_i|, av = 2^-8
   sum_i P_ij |dO_i|. */
void orc_attn_bwd_values(const double* Q, const double* K, const double* V, const double* O, const double* dO,
                         const double* lse, int B, int S, int Hq, int Hkv, int D, double scale,
                         const int32_t* qrows, int nq, const int32_t* krows, int nk, double* dq, double* dk,
                         double* dv, double* aq, double* ak, double* av) {
  const double u = ldexp(1.0, -8);
  const int G = Hq / Hkv;
  double* delta = (double*)malloc(sizeof(double) * (int64_t)B * Hq * S);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < (int64_t)B * Hq * S; ++r) delta[r] = dot(dO + r * D, O + r * D, D);
  if (dq) {
#pragma omp parallel for collapse(3) schedule(dynamic, 4)
    for (int b = 0; b < B; ++b)
      for (int hq = 0; hq < Hq; ++hq)
        for (int r = 0; r < nq; ++r) {
          const int i = row_index(qrows, r), hk = hq / G;
          const int64_t qi = (((int64_t)b * Hq + hq) * S + i);
          const double* Kh = K + ((int64_t)b * Hkv + hk) * S * D;
          const double* Vh = V + ((int64_t)b * Hkv + hk) * S * D;
          double* out = dq + (((int64_t)b * Hq + hq) * nq + r) * D;
          double* al = aq ? aq + (((int64_t)b * Hq + hq) * nq + r) * D : NULL;
          for (int d = 0; d < D; ++d) out[d] = 0.0;
          if (al)
            for (int d = 0; d < D; ++d) al[d] = 0.0;
          for (int j = 0; j <= i; ++j) {
            const double p = exp(scale * dot(Q + qi * D, Kh + (int64_t)j * D, D) - lse[qi]);
            const double ds = p * (dot(dO + qi * D, Vh + (int64_t)j * D, D) - delta[qi]);
            for (int d = 0; d < D; ++d) out[d] += ds * Kh[(int64_t)j * D + d];
            if (al)
              for (int d = 0; d < D; ++d) al[d] += fabs(ds * Kh[(int64_t)j * D + d]);
          }
          for (int d = 0; d < D; ++d) out[d] *= scale;
          if (al)
            for (int d = 0; d < D; ++d) al[d] *= u * scale;
        }
  }
  if (dk || dv) {
#pragma omp parallel for collapse(3) schedule(dynamic, 4)
    for (int b = 0; b < B; ++b)
      for (int hk = 0; hk < Hkv; ++hk)
        for (int r = 0; r < nk; ++r) {
          const int j = row_index(krows, r);
          const double* kj = K + (((int64_t)b * Hkv + hk) * S + j) * D;
          const double* vj = V + (((int64_t)b * Hkv + hk) * S + j) * D;
          double* ak_ = (double*)calloc(D, sizeof(double));
          double* av_ = (double*)calloc(D, sizeof(double));
          double* bk = (double*)calloc(D, sizeof(double));
          double* bv = (double*)calloc(D, sizeof(double));
          for (int hq = hk * G; hq < (hk + 1) * G; ++hq)
            for (int i = j; i < S; ++i) {
              const int64_t qi = (((int64_t)b * Hq + hq) * S + i);
              const double p = exp(scale * dot(Q + qi * D, kj, D) - lse[qi]);
              const double ds = p * (dot(dO + qi * D, vj, D) - delta[qi]);
              for (int d = 0; d < D; ++d) {
                av_[d] += p * dO[qi * D + d];
                ak_[d] += ds * Q[qi * D + d];
                bv[d] += fabs(p * dO[qi * D + d]);
                bk[d] += fabs(ds * Q[qi * D + d]);
              }
            }
          const int64_t orow = (((int64_t)b * Hkv + hk) * nk + r) * D;
          for (int d = 0; d < D; ++d) {
            if (dk) dk[orow + d] = scale * ak_[d];
            if (dv) dv[orow + d] = av_[d];
            if (ak) ak[orow + d] = u * scale * bk[d];
            if (av) av[orow + d] = u * bv[d];
          }
          free(ak_);
          free(av_);
          free(bk);
          free(bv);
        }
  }
  free(delta);
}

/* The same from the codes in the library's layouts: Q, K decoded from their
   rowwise MXFP8 bytes (O4/O3), V from the token-normalised copy (O6/O3); O and
   dO bf16 [B,S,Hq,D] views, lse fp32 [B,Hq,S]. */
void orc_attn_bwd(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks, const uint8_t* vt,
                  const uint8_t* vta, const uint16_t* o, int64_t osb, int64_t oss, int64_t osh, const float* lse,
                  const uint16_t* dout, int64_t gsb, int64_t gss, int64_t gsh, int B, int S, int Hq, int Hkv, int D,
                  float scale, const int32_t* qrows, int nq, const int32_t* krows, int nk, double* dq, double* dk,
                  double* dv, double* aq, double* ak, double* av) {
  double* Q = decode_rowwise(qc, qs, B, Hq, S, D);
  double* K = decode_rowwise(kc, ks, B, Hkv, S, D);
  double* V = decode_vtn(vt, vta, B, Hkv, S, D);
  double* Ov = bf16_tensor(o, osb, oss, osh, B, S, Hq, D);
  double* dOv = bf16_tensor(dout, gsb, gss, gsh, B, S, Hq, D);
  double* L = (double*)malloc(sizeof(double) * (int64_t)B * Hq * S);
  for (int64_t r = 0; r < (int64_t)B * Hq * S; ++r) L[r] = (double)lse[r];
  orc_attn_bwd_values(Q, K, V, Ov, dOv, L, B, S, Hq, Hkv, D, (double)scale, qrows, nq, krows, nk, dq, dk, dv, aq,
                      ak, av);
  free(Q);
  free(K);
  free(V);
  free(Ov);
  free(dOv);
  free(L);
}
