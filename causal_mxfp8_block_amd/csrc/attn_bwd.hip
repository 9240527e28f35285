// attn_bwd.hip -- backward of leak-free causal MXFP8 attention on decoded operands, gfx950.
//
// TransformerEngine PR #3865, "Description", backward bullet: the backward runs in BF16 on Q/K decoded
// from their rowwise MXFP8 bytes and V decoded from the token-normalised copy, so no gradient depends
// on a later token through a shared scale. With the forward's O and LSE as the softmax statistics:
//   Delta_i = dO_i . O_i,   P_ij = exp(scale Q_i.K_j - lse_i) (j <= i),   dS_ij = P_ij (dO_i.V_j - Delta_i)
//   dQ_i = scale sum_j dS_ij K_j,   dK_j = scale sum_i dS_ij Q_i,   dV_j = sum_i P_ij dO_i
// (dK, dV summed over the query heads of a KV head).
//
// Design (CDNA4, wave64, bf16 MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//  * A preparation pass decodes Q, K and V to bf16 (exact: an E4M3 value times a power of two has 4
//    significant bits) and copies dO, each head-major, plus a transposed [D][S] copy of Q, K and dO
//    for the MFMA operands that contract over tokens; it also forms Delta.
//  * dK/dV kernel: one wave per 32 keys, one wave per SIMD (its 512 registers hold the K and V
//    operands, both accumulators and a whole pipelined step). For every query head of the KV head and
//    every 32-query block at or after the keys, it computes S = Q K^T and dP = dO V^T (keys on the
//    lanes, queries on the accumulator elements), P and dS elementwise, and accumulates
//    dV^T += dO^T P and dK^T += Q^T dS. P and dS are the B operand of those MFMAs straight from the
//    accumulator layout: the accumulator's query order is a permutation of the B operand's
//    contraction order, and the A operand (dO^T, Q^T, read from LDS) is stored in the same permuted
//    order. The steps are software-pipelined.
//  * dQ kernel: one wave per 32 queries, their Q and dO operands in registers; 8 waves (256 queries)
//    per workgroup and one workgroup per CU (two waves per SIMD), so that each K/V tile brought into LDS
//    serves 256 queries: what the tiles cost is the data moved from L2, not its latency. For
//    every 32-key block at or before the queries it computes S^T = K Q^T and dP^T = V dO^T (queries on
//    the lanes: lse and Delta are per-lane scalars) and accumulates dQ^T += K^T dS^T the same way,
//    pipelined by one block: the dQ products of a block are issued behind the S and dP products of the
//    next one, and that block's P and dS are formed while they run.
//  * Key > query is masked to P = 0, only on the steps that straddle the diagonal. The loops start at
//    the workgroup's first block on or below the diagonal, so a wave whose own blocks start later
//    computes at most three (dK/dV) or seven (dQ) fully masked steps.
//  * Query (dK/dV) and key (dQ) blocks go from global memory straight into LDS rings shared by the
//    workgroup (loads with the LDS flag; no register staging). Rows are unpadded and the 16-byte
//    chunks XOR-swizzled, so the operand reads are bank-conflict-free; the preparation pass writes the
//    transposed copies in the MFMA slot order. Both grids run the longest workgroups first.
#include "device_common.h"
#include "launch.h"

#include <type_traits>

namespace mxfa {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int BW_ROW = 136;  // LDS pitch (bf16) of the preparation pass's [token][D] tile: 128 + 8 pad

__device__ __forceinline__ v8bf ld8bf(const uint16_t* p) {  // 16 bytes, 16-byte aligned
  return __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ v16f mfma_bf16(const v8bf& a, const v8bf& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// Elements 8t .. 8t+7 of an accumulator as bf16 (round to nearest even).
__device__ __forceinline__ v8bf to_bf16(const v16f& x, int t) {
  v8bf r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[8 * t + e];
  return r;
}

// Position of token q (0..31) of a transposed tile row in the MFMA slot order of both kernels'
// 32x32x16 operands: within each 16-token half, bits 2 and 3 swapped, so that lane half h reads tokens
// 4h..4h+3 and 8+4h..8+4h+3 of the half as one 16-byte operand (the accumulator's row order).
__device__ __forceinline__ int dq_tpos(int q) { return (q & 16) | ((q & 4) << 1) | ((q & 8) >> 1) | (q & 3); }

// ---- preparation -------------------------------------------------------------------------------
// One workgroup per (b, h, 64-token tile), 256 threads: thread g handles token g/4, columns
// 32(g%4) .. +32. Source kSrc: 0 rowwise codes + E8M0 per 32 columns, 1 token-normalised codes + one
// E8M0 amplitude per token, 2 a bf16 [B,S,H,D] view (with Delta from the o view and lse * log2(e)
// from lse when delta != null). Writes the bf16 rows to out [B,H,S,D] and, when out_t != null, the
// transposed out_t [B,H,D,S]; with kSlot 1 the tokens of each 32-token block of out_t are stored in the
// MFMA slot order, dq_tpos, so that the tiles load as contiguous 16-byte pieces.
template <int kSrc, int kSlot = 0>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint8_t* codes, const uint8_t* scales, const uint16_t* x,
                                                       int64_t sb, int64_t ss, int64_t sh, const uint16_t* o,
                                                       int64_t osb, int64_t oss, int64_t osh, int S, int H,
                                                       uint16_t* out, uint16_t* out_t, float* delta,
                                                       const float* lse = nullptr, float* lse2 = nullptr) {
  __shared__ __align__(16) uint16_t tile[64 * BW_ROW];
  const int g = threadIdx.x, tok = g >> 2, c0 = (g & 3) * 32;
  const int s0 = blockIdx.x * 64, h = blockIdx.y, b = blockIdx.z;
  const int s = s0 + tok;
  const int64_t bh = (int64_t)b * H + h;
  uint32_t w[16];  // 32 bf16, packed in pairs
  if (s < S) {
    if (kSrc == 2) {
      const uint16_t* row = x + b * sb + (int64_t)s * ss + h * sh + c0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = reinterpret_cast<const uint4*>(row)[q];
        w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
      }
      if (delta) {
        const uint16_t* orow = o + b * osb + (int64_t)s * oss + h * osh + c0;
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = reinterpret_cast<const uint4*>(orow)[q];
          const uint32_t ov[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t gw = w[4 * q + e];
            acc = fmaf(bf16_to_f32(gw & 0xffffu), bf16_to_f32(ov[e] & 0xffffu), acc);
            acc = fmaf(bf16_to_f32(gw >> 16), bf16_to_f32(ov[e] >> 16), acc);
          }
        }
        acc += __shfl_xor(acc, 1);
        acc += __shfl_xor(acc, 2);
        if ((g & 3) == 0) {
          delta[bh * S + s] = acc;
          lse2[bh * S + s] = lse[bh * S + s] * 1.4426950408889634f;
        }
      }
    } else {
      const uint8_t* crow = codes + (bh * S + s) * 128 + c0;
      const float sc = kSrc == 0 ? e8m0_to_f32(scales[(bh * S + s) * 4 + (g & 3)]) : e8m0_to_f32(scales[bh * S + s]);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4 v = reinterpret_cast<const uint4*>(crow)[q];
        const uint32_t cw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // E4M3 value times a power of two has at most 4 significant bits: its top 16 bits are the bf16
          const uint32_t lo0 = f2u(e4m3_to_f32(cw[e] & 0xffu) * sc) >> 16;
          const uint32_t hi0 = f2u(e4m3_to_f32((cw[e] >> 8) & 0xffu) * sc) >> 16;
          const uint32_t lo1 = f2u(e4m3_to_f32((cw[e] >> 16) & 0xffu) * sc) >> 16;
          const uint32_t hi1 = f2u(e4m3_to_f32(cw[e] >> 24) * sc) >> 16;
          w[8 * q + 2 * e] = lo0 | (hi0 << 16);
          w[8 * q + 2 * e + 1] = lo1 | (hi1 << 16);
        }
      }
    }
    uint4* dst = reinterpret_cast<uint4*>(out + (bh * S + s) * 128 + c0);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
  }
  if (!out_t) return;
  uint4* trow = reinterpret_cast<uint4*>(tile + tok * BW_ROW + c0);
#pragma unroll
  for (int q = 0; q < 4; ++q) trow[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
  __syncthreads();
  // transposed: thread g writes column d = g/2, tokens 32(g%2) .. +32 of this tile
  const int d = g >> 1, t0 = (g & 1) * 32;
  if (s0 + t0 >= S) return;  // S % 32 == 0: a half tile is either wholly inside or wholly outside
  uint32_t p[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    // tokens t0 + 2e and t0 + 2e + 1 stay one dword (both orders keep even-odd pairs together)
    const int pos = kSlot == 1 ? (dq_tpos(2 * e) >> 1) : e;
    p[pos] = (uint32_t)tile[(t0 + 2 * e) * BW_ROW + d] | ((uint32_t)tile[(t0 + 2 * e + 1) * BW_ROW + d] << 16);
  }
  uint4* tdst = reinterpret_cast<uint4*>(out_t + (bh * 128 + d) * S + s0 + t0);
#pragma unroll
  for (int q = 0; q < 4; ++q) tdst[q] = make_uint4(p[4 * q], p[4 * q + 1], p[4 * q + 2], p[4 * q + 3]);
}

struct BwdParams {
  const uint16_t *qd, *qdt, *kd, *kdt, *vd, *gd, *gdt;  // decoded operands (workspace)
  const float *lse, *delta;                              // [B,Hq,S]
  const float* lse2;                                     // lse * log2(e), [B,Hq,S] (workspace)
  int B, S, Hq, Hkv;
  float scale, scale_log2;
  uint16_t *dq, *dk, *dv;                                // bf16 outputs (views)
  int64_t qsb, qss, qsh, ksb, kss, ksh;                 // strides of dq and of dk/dv
};

// ---- dK, dV ------------------------------------------------------------------------------------
// Global -> LDS without registers: lane l's 16 (or 4) bytes land at lds + 16 l (4 l); lds wave-uniform.
__device__ __forceinline__ void gload_lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)g, (__attribute__((address_space(3))) void*)lds,
                                   16, 0, 0);
}
__device__ __forceinline__ void gload_lds4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)g, (__attribute__((address_space(3))) void*)lds,
                                   4, 0, 0);
}

// The same loads written out, for loops that keep several iterations' loads in flight: the compiler
// does not see them, so it neither counts them in its waits nor makes every LDS read wait for them (it
// cannot tell the slots apart across iterations); the loop waits for them itself. Address = a scalar
// base plus a 32-bit per-lane byte offset; M0 holds the LDS address, set by the compiler through the
// operand constraint; the nop is the wait state an LDS DMA needs after an M0 write. No register is
// written, so nothing of the instruction stays in flight in a register.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void dma_lds16(const void* base, uint32_t voff, void* lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds_addr(lds)) : "memory");
}
__device__ __forceinline__ void dma_lds4(const void* base, uint32_t voff, void* lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds_addr(lds)) : "memory");
}

// Workgroup: 4 waves, one per SIMD, = keys 128 kt .. 128 kt + 127 of (b, hk); wave w owns keys
// 128 kt + 32 w + [0, 32), its K and V rows held in registers as B operands and its dK^T and dV^T
// accumulators (128 x 32 each) in registers. 32 keys per wave let every Q and dO element read from LDS
// feed 32 keys of each product, half the LDS traffic per FLOP of a 16-key wave. Steps n = (query head,
// 32-query block), the blocks from the last one down to 4kt. Per step, with the keys on the MFMA
// columns (v_mfma_f32_32x32x16_bf16: A lane (m = l%32, g = l/32) element e <-> A[m][8g+e]; B lane
// (n = l%32, g) element e <-> B[8g+e][n]; C lane (n, g) element i <-> C[8(i/4) + 4g + i%4][n]):
// S = Q K^T and dP = dO V^T (K = D in eight 16-wide steps), P and dS elementwise in the accumulators
// (lane: key l%32, element i: query 8(i/4) + 4g + i%4), then dV^T += dO^T P and dK^T += Q^T dS, two
// 16-query slices each, with P and dS as the B operand straight from the accumulators: slot (g, e) of
// slice t is accumulator element 8t + e, query 16t + 8(e/4) + 4g + e%4 (dq_tpos, the order in which
// the preparation pass stores the transposed copies). The loop is software-pipelined: in iteration i
// the VALU computes P and dS of step i while the matrix core runs the S and dP products of step i + 1
// and the dV and dK products of step i - 1. The tiles go from global memory straight into LDS (loads
// with the LDS flag) in three rings, each as far ahead as its slots allow: the Q and dO rows of step
// i + 4 (read in iteration i + 3), the transposed tiles of step i + 2 (read in iteration i + 3) and the
// lse and Delta of step i + 3 (read in iteration i + 3); so every load has two iterations to arrive,
// and an iteration ends by waiting only for the loads issued two iterations before. Every iteration
// issues the same loads (past the last step they repeat it into a free slot), which keeps that count
// exact. One wave per SIMD issues every instruction of its step itself, so the step keeps them few:
// the load addresses advance by scalar increments, the causal mask costs nothing off the diagonal
// (on a diagonal step a masked pair gets lse = +inf, hence P = 0 and dS = 0), and P and dS go to
// bf16 as they are formed.
constexpr int DKDV_NBUF = 4;
struct DkdvRows {    // Q, dO rows: chunk x of row r in slot x ^ (r & 15) (unpadded, conflict-free reads)
  uint16_t q[32 * 128], g[32 * 128];
};
struct DkdvTrans {   // Q^T, dO^T rows in slot order: chunk x of row d in slot x ^ ((d >> 2) & 3)
  uint16_t qt[128 * 32], gt[128 * 32];
};
struct DkdvStats {   // lse * log2(e) and Delta of the step's 32 queries
  float l[32], d[32];
};
constexpr int DKDV_LOADS_PER_ITER = 9;  // per thread: 4 row chunks, 4 transposed chunks, 1 stats word

// Scalar position of the load streams in the step sequence. Step j is query head hk G + j / per_head,
// 32-query block nqb - 1 - j % per_head; x = (b Hq + head) S + q0 and t = (b Hq + head) 128 S + q0 are
// the element offsets of its Q/dO rows (x 128), its transposed columns (t) and its lse/Delta (x).
struct DkdvStream {
  int64_t x, t;
  int left;   // steps of the current head from j on
  int j;
};
__device__ __forceinline__ void dkdv_advance(DkdvStream& s, int nsteps, int per_head, int S) {
  if (s.j + 1 >= nsteps) return;  // past the last step the loads repeat it
  ++s.j;
  const bool wrap = --s.left == 0;
  s.left = wrap ? per_head : s.left;
  s.x += wrap ? (int64_t)S + 32 * (per_head - 1) : -32;
  s.t += wrap ? (int64_t)128 * S + 32 * (per_head - 1) : -32;
}
// Per-lane byte offsets of a thread's chunks: thread tid fills LDS chunks 256 i + tid (i = 0, 1; 16
// bytes each; each wave's 64 chunks of one instruction are contiguous) of each tile: of Q and dO, row
// r = c/16, slot c%16, holding chunk (c%16) ^ (r & 15) of that query's row; of Q^T and dO^T, row
// d = c/4, slot c%4, holding chunk (c%4) ^ ((d >> 2) & 3) of the block's 64 bytes of row d (S <= 2^24
// keeps 2 (127 S + 24) below 2^32). The lse and Delta words come in a quarter per wave (lanes
// 16w .. 16w + 15 of wave w), so that every thread issues the same number of loads.
struct DkdvLanes {
  uint32_t roff[2], toff[2], soff;
  bool sl;  // this lane loads a stats word
};
// One iteration's loads (rows of one step, transposed tiles of another, stats of a third), issued in
// nine parts so that they can be spread over the iteration: part k < 8 is one 16-byte chunk per thread
// of a tile, part 8 the stats word.
struct DkdvLoads {
  const uint16_t *qr, *gr, *qt, *gt;
  const void* sb;
  DkdvRows* __restrict__ R;
  DkdvTrans* __restrict__ T;
  DkdvStats* __restrict__ St;
  __device__ __forceinline__ DkdvLoads(const BwdParams& P, int64_t xr, int64_t tt, int64_t xs, DkdvRows* R_,
                                       DkdvTrans* T_, DkdvStats* St_, int wave_u)
      : qr(P.qd + xr * 128), gr(P.gd + xr * 128), qt(P.qdt + tt), gt(P.gdt + tt),
        sb(wave_u < 2 ? (const void*)(P.lse2 + xs) : (const void*)(P.delta + xs - 32)), R(R_), T(T_), St(St_) {}
  __device__ __forceinline__ void part(int k, const DkdvLanes& L, int wave_u) const {
    const int i = k & 1, lo = 16 * (256 * i + 64 * wave_u);
    if (k < 2) dma_lds16(qr, L.roff[i], reinterpret_cast<uint8_t*>(R->q) + lo);
    else if (k < 4) dma_lds16(gr, L.roff[i], reinterpret_cast<uint8_t*>(R->g) + lo);
    else if (k < 6) dma_lds16(qt, L.toff[i], reinterpret_cast<uint8_t*>(T->qt) + lo);
    else if (k < 8) dma_lds16(gt, L.toff[i], reinterpret_cast<uint8_t*>(T->gt) + lo);
    else if (L.sl) dma_lds4(sb, L.soff, St->l);
  }
  __device__ __forceinline__ void all(const DkdvLanes& L, int wave_u) const {
#pragma unroll
    for (int k = 0; k < 9; ++k) part(k, L, wave_u);
  }
};

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {  // round to nearest even
  const v2bf r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
}

// One iteration of the pipelined dK/dV loop (see above). The LDS slots are restrict pointers. Past the
// last step Rn is a stale slot (its products are unused). P and dS of step st (bf16 pairs of
// accumulator elements 2k, 2k + 1) replace those of step st - 1 (pw, sw) at the end.
__device__ __forceinline__ void dkdv_pipe_iter(const DkdvLoads& ld, const DkdvLanes& Ln, int wave_u,
                                               const DkdvRows* __restrict__ Rn, const DkdvTrans* __restrict__ Tp,
                                               const DkdvStats* __restrict__ Sc, int koff, int n, int g,
                                               float scale_log2, const v8bf (&kop)[8], const v8bf (&vop)[8],
                                               v16f (&dkT)[4], v16f (&dvT)[4], const v16f& sc, const v16f& pc,
                                               v16f& sn, v16f& pn, uint32_t (&pw)[8], uint32_t (&sw)[8]) {
  ld.part(8, Ln, wave_u);
  float lv[16], dv[16];  // element i: query 8(i/4) + 4g + i%4
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float4 l4 = *reinterpret_cast<const float4*>(Sc->l + 8 * j + 4 * g);
    const float4 d4 = *reinterpret_cast<const float4*>(Sc->d + 8 * j + 4 * g);
    lv[4 * j] = l4.x; lv[4 * j + 1] = l4.y; lv[4 * j + 2] = l4.z; lv[4 * j + 3] = l4.w;
    dv[4 * j] = d4.x; dv[4 * j + 1] = d4.y; dv[4 * j + 2] = d4.z; dv[4 * j + 3] = d4.w;
  }
  if (koff > -31) {  // a key of this wave may lie after a query of the block: mask through lse
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (n + koff > 8 * (i >> 2) + 4 * g + (i & 3)) lv[i] = INFINITY;
  }
  // Operands of group k: row n of Q and dO, columns 16k + 8g (chunk 2k + g); row 32(k/2) + n of the
  // transposes, slots 16(k%2) + 8g (chunk 2(k%2) + g).
  auto rowoff = [&](int k) { return n * 128 + 8 * ((2 * k + g) ^ (n & 15)); };
  auto troff = [&](int k) { return (32 * (k >> 1) + n) * 32 + 8 * ((2 * (k & 1) + g) ^ ((n >> 2) & 3)); };
  v8bf qa = ld8bf(Rn->q + rowoff(0)), ga = ld8bf(Rn->g + rowoff(0));
  v8bf gta = ld8bf(Tp->gt + troff(0)), qta = ld8bf(Tp->qt + troff(0));
  uint32_t npw[8], nsw[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    v8bf qa2, ga2, gta2, qta2;
    if (k < 7) {  // the next group's operands, read one group ahead
      qa2 = ld8bf(Rn->q + rowoff(k + 1));
      ga2 = ld8bf(Rn->g + rowoff(k + 1));
      gta2 = ld8bf(Tp->gt + troff(k + 1));
      qta2 = ld8bf(Tp->qt + troff(k + 1));
    }
    ld.part(k, Ln, wave_u);
    sn = k == 0 ? mfma_bf16(qa, kop[0], v16f{}) : mfma_bf16(qa, kop[k], sn);
    pn = k == 0 ? mfma_bf16(ga, vop[0], v16f{}) : mfma_bf16(ga, vop[k], pn);
    {
      const int t = k & 1;
      const v8bf pb = __builtin_bit_cast(v8bf, uint4{pw[4 * t], pw[4 * t + 1], pw[4 * t + 2], pw[4 * t + 3]});
      const v8bf sb = __builtin_bit_cast(v8bf, uint4{sw[4 * t], sw[4 * t + 1], sw[4 * t + 2], sw[4 * t + 3]});
      dvT[k >> 1] = mfma_bf16(gta, pb, dvT[k >> 1]);
      dkT[k >> 1] = mfma_bf16(qta, sb, dkT[k >> 1]);
    }
    {  // P and dS of elements 2k, 2k + 1 of step st (query 8(i/4) + 4g + i%4, key key0 + n)
      const int i = 2 * k;
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[i], scale_log2, -lv[i]));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[i + 1], scale_log2, -lv[i + 1]));
      npw[k] = pack_bf16(p0, p1);
      nsw[k] = pack_bf16(p0 * (pc[i] - dv[i]), p1 * (pc[i + 1] - dv[i + 1]));
    }
    if (k < 7) {
      qa = qa2; ga = ga2; gta = gta2; qta = qta2;
    }
    // Issue order of the group: the next group's four operand reads, then the four MFMAs with the
    // VALU work between them (the compiler would otherwise read each operand just before its MFMA).
    if (k == 0) __builtin_amdgcn_sched_group_barrier(0x0100, 4, 0);
    if (k < 7) __builtin_amdgcn_sched_group_barrier(0x0100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x0002, 3, 0);
    __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x0002, 3, 0);
    __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x0002, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x0002, 2, 0);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    pw[e] = npw[e];
    sw[e] = nsw[e];
  }
  // Iteration st + 1 reads the loads issued in iteration st - 2 (or before the loop): wait until at
  // most the last two iterations' loads are in flight; the barrier publishes them.
  static_assert(2 * DKDV_LOADS_PER_ITER <= 63, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * DKDV_LOADS_PER_ITER & 15) | ((2 * DKDV_LOADS_PER_ITER >> 4) << 14));
  __syncthreads();
}

__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dkdv_kernel(const BwdParams P) {
  __shared__ __align__(16) DkdvRows rows[DKDV_NBUF];
  __shared__ __align__(16) DkdvTrans trans[DKDV_NBUF];
  __shared__ __align__(16) DkdvStats stats[DKDV_NBUF];
  const int S = P.S, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 31, g = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // Longest first: id / (Hkv B) is the key tile (tile kt has the most query blocks at kt = 0).
  const int nbh = P.Hkv * P.B, id = (int)blockIdx.x;
  const int kt = id / nbh, bh = id - kt * nbh, b = bh / P.Hkv, hk = bh - b * P.Hkv;
  const int G = P.Hq / P.Hkv;
  const int key0 = 128 * kt + 32 * wave, key0_u = 128 * kt + 32 * wave_u;
  const bool valid = key0 < S;  // S % 32 == 0: a wave's 32 keys are all inside or all outside
  const int64_t bhk = (int64_t)b * P.Hkv + hk;
  // B operands: lane (key n, g), step s holds columns 16s + 8g + [0, 8) of the key's K and V rows.
  v8bf kop[8], vop[8];
  const int krow = valid ? key0 + n : 0;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    kop[s] = ld8bf(P.kd + (bhk * S + krow) * 128 + 16 * s + 8 * g);
    vop[s] = ld8bf(P.vd + (bhk * S + krow) * 128 + 16 * s + 8 * g);
  }
  v16f dkT[4], dvT[4];  // tile dt: lane (key n, g), element i <-> column d = 32dt + 8(i/4) + 4g + i%4
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dkT[dt][i] = dvT[dt][i] = 0.f;
  const int nqb = S / 32, qb0 = 4 * kt, per_head = nqb - qb0, nsteps = G * per_head;
  DkdvLanes L;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = 256 * i + tid, r = c >> 4, x = (c & 15) ^ (r & 15), d = c >> 2, xt = (c & 3) ^ ((d >> 2) & 3);
    L.roff[i] = 2u * (uint32_t)(r * 128 + 8 * x);
    L.toff[i] = 2u * ((uint32_t)d * (uint32_t)S + 8u * (uint32_t)xt);
  }
  L.soff = 4u * (uint32_t)lane;  // words 0..31 lse, 32..63 Delta (the Delta base is 32 words lower)
  L.sl = (lane >> 4) == wave;
  // Load streams: rows of step i + 4, transposed of step i + 2, stats of step i + 3 in iteration i.
  DkdvStream st;
  st.j = 0;
  st.left = per_head;
  st.x = ((int64_t)b * P.Hq + hk * G) * S + 32 * (nqb - 1);
  st.t = ((int64_t)b * P.Hq + hk * G) * 128 * S + 32 * (nqb - 1);
  // Transposed slot 3 stands in for step -1 in iteration 0: zero tiles, which with zero P and dS add
  // exactly 0. Step 3 first arrives there in iteration 1.
  {
    uint4* z0 = reinterpret_cast<uint4*>(trans[DKDV_NBUF - 1].qt);
    uint4* z1 = reinterpret_cast<uint4*>(trans[DKDV_NBUF - 1].gt);
#pragma unroll
    for (int i = 0; i < 2; ++i) z0[256 * i + tid] = z1[256 * i + tid] = uint4{0u, 0u, 0u, 0u};
  }
  // Before the loop: rows of steps 0..3, transposed of steps 0, 1, stats of steps 0..2 (the stream
  // positions of steps 0..4 pass by; the loop starts with rows at 4, stats at 3, transposed at 2).
  int64_t x3, t2, t3;
  {
    int64_t xs[4], ts[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xs[j] = st.x; ts[j] = st.t;
      dkdv_advance(st, nsteps, per_head, S);
    }
    // steps 2 and 3 bring transposed tiles the loop loads again (into slot 2, reloaded in iteration 0;
    // slot 3 keeps its zeros) and step 3 stats the loop loads again
    DkdvLoads(P, xs[0], ts[0], xs[0], &rows[0], &trans[0], &stats[0], wave_u).all(L, wave_u);
    DkdvLoads(P, xs[1], ts[1], xs[1], &rows[1], &trans[1], &stats[1], wave_u).all(L, wave_u);
    DkdvLoads(P, xs[2], ts[2], xs[2], &rows[2], &trans[2], &stats[2], wave_u).all(L, wave_u);
    DkdvLoads(P, xs[3], ts[3], xs[3], &rows[3], &trans[2], &stats[3], wave_u).all(L, wave_u);
    x3 = xs[3]; t2 = ts[2]; t3 = ts[3];
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  // S and dP of step 0
  v16f sa, pa, sb2, pb2;
#pragma unroll
  for (int i = 0; i < 16; ++i) sa[i] = pa[i] = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int off = n * 128 + 8 * ((2 * s + g) ^ (n & 15));
    sa = mfma_bf16(ld8bf(rows[0].q + off), kop[s], sa);
    pa = mfma_bf16(ld8bf(rows[0].g + off), vop[s], pa);
  }
  uint32_t pw[8], sw[8];  // P and dS of the previous step as bf16 pairs (none before step 0)
#pragma unroll
  for (int e = 0; e < 8; ++e) pw[e] = sw[e] = 0u;
  // unrolled by four: ring slots are constants (step i in slot i % 4); S and dP buffers alternate
  auto it4 = [&](auto kslot, int i, v16f& sc, v16f& pc, v16f& sn, v16f& pn) {
    constexpr int s = decltype(kslot)::value;
    const DkdvLoads ld(P, st.x, t2, x3, &rows[s], &trans[(s + 2) % DKDV_NBUF], &stats[(s + 3) % DKDV_NBUF], wave_u);
    t2 = t3; t3 = st.t; x3 = st.x;
    dkdv_advance(st, nsteps, per_head, S);
    const int qb = nqb - 1 - i % per_head;
    dkdv_pipe_iter(ld, L, wave_u, &rows[(s + 1) % DKDV_NBUF], &trans[(s + 3) % DKDV_NBUF], &stats[s], key0_u - 32 * qb, n, g,
                   P.scale_log2, kop, vop, dkT, dvT, sc, pc, sn, pn, pw, sw);
  };
  for (int i = 0; i < nsteps; i += 4) {
    it4(std::integral_constant<int, 0>{}, i, sa, pa, sb2, pb2);
    if (i + 1 < nsteps) it4(std::integral_constant<int, 1>{}, i + 1, sb2, pb2, sa, pa);
    if (i + 2 < nsteps) it4(std::integral_constant<int, 2>{}, i + 2, sa, pa, sb2, pb2);
    if (i + 3 < nsteps) it4(std::integral_constant<int, 3>{}, i + 3, sb2, pb2, sa, pa);
  }
  // Every load has landed (also the repeats past the last step, which must not outlive the workgroup).
  __builtin_amdgcn_s_waitcnt(0x0F70);
  {  // dV and dK of the last step
    const DkdvTrans& Tp = trans[(nsteps - 1) % DKDV_NBUF];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int off = (32 * (k >> 1) + n) * 32 + 8 * ((2 * (k & 1) + g) ^ ((n >> 2) & 3));
      const int t = k & 1;
      const v8bf pb = __builtin_bit_cast(v8bf, uint4{pw[4 * t], pw[4 * t + 1], pw[4 * t + 2], pw[4 * t + 3]});
      const v8bf sb = __builtin_bit_cast(v8bf, uint4{sw[4 * t], sw[4 * t + 1], sw[4 * t + 2], sw[4 * t + 3]});
      dvT[k >> 1] = mfma_bf16(ld8bf(Tp.gt + off), pb, dvT[k >> 1]);
      dkT[k >> 1] = mfma_bf16(ld8bf(Tp.qt + off), sb, dkT[k >> 1]);
    }
  }
  if (!valid) return;
  // lane (key n, g), element i of tile dt: column 32dt + 8(i/4) + 4g + i%4
  const int64_t off = b * P.ksb + (int64_t)(key0 + n) * P.kss + hk * P.ksh + 4 * g;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint2 pk, pv;
      pk.x = f32_to_bf16(dkT[dt][4 * j] * P.scale) | (f32_to_bf16(dkT[dt][4 * j + 1] * P.scale) << 16);
      pk.y = f32_to_bf16(dkT[dt][4 * j + 2] * P.scale) | (f32_to_bf16(dkT[dt][4 * j + 3] * P.scale) << 16);
      pv.x = f32_to_bf16(dvT[dt][4 * j]) | (f32_to_bf16(dvT[dt][4 * j + 1]) << 16);
      pv.y = f32_to_bf16(dvT[dt][4 * j + 2]) | (f32_to_bf16(dvT[dt][4 * j + 3]) << 16);
      *reinterpret_cast<uint2*>(P.dk + off + 32 * dt + 8 * j) = pk;
      *reinterpret_cast<uint2*>(P.dv + off + 32 * dt + 8 * j) = pv;
    }
}

// ---- dQ ----------------------------------------------------------------------------------------
// Workgroup: 8 waves = queries 256 qt .. 256 qt + 255 of (b, hq); wave w owns queries 32(8qt + w) + [0, 32).
// Key blocks go from global memory straight into a ring of three LDS slots (loads with the LDS flag),
// one block ahead. The loop is software-pipelined by one stage: iteration kb issues the S^T and dP^T
// products of block kb, then the dQ^T products of block kb - 1 (from that block's K^T tile, still in
// its slot, and its dS kept as bf16 pairs), and forms P and dS of block kb on the VALU while those run;
// so a wave's VALU work no longer waits behind its own dQ products.
struct DqTiles {
  uint16_t k[32 * 128], v[32 * 128];  // K, V rows: chunk c of row r in slot c ^ (r & 15)
  uint16_t kt[128 * 32];              // K^T rows (dQ slot order): chunk c of row d in slot c ^ ((d >> 2) & 3)
};
constexpr int DQ_NBUF = 3;
__global__ __launch_bounds__(512, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(const BwdParams P) {
  __shared__ __align__(16) DqTiles buf[DQ_NBUF];
  const int S = P.S, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 31, h = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // Longest first: the last query tile (the most key blocks) of every (b, hq) comes first.
  const int nbh = P.Hq * P.B, id = (int)blockIdx.x, ntiles = (S + 255) / 256;
  const int qt = ntiles - 1 - id / nbh, bh = id - (id / nbh) * nbh, b = bh / P.Hq, hq = bh - b * P.Hq;
  const int hk = hq / (P.Hq / P.Hkv);
  const int qb = 8 * qt + wave, q0 = 32 * qb;
  const bool valid = q0 < S;
  const int64_t bhq = (int64_t)b * P.Hq + hq, bhk = (int64_t)b * P.Hkv + hk;
  // This wave's Q and dO rows as B operands: lane (query c, h), step s holds columns 16s + 8h + [0, 8).
  v8bf qop[8], gop[8];
  const int qrow = valid ? q0 + c : 0;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    qop[s] = ld8bf(P.qd + (bhq * S + qrow) * 128 + 16 * s + 8 * h);
    gop[s] = ld8bf(P.gd + (bhq * S + qrow) * 128 + 16 * s + 8 * h);
  }
  const float lse2 = P.lse[bhq * S + qrow] * 1.4426950408889634f, del = P.delta[bhq * S + qrow];
  v16f dqT[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqT[dt][i] = 0.f;
  const uint16_t *kd = P.kd + bhk * S * 128, *vd = P.vd + bhk * S * 128, *kdt = P.kdt + bhk * 128 * S;
  const int nkb = min(8 * qt + 7, S / 32 - 1) + 1;  // key blocks any wave of the workgroup needs
  // Thread tid (of 512) fills LDS chunk ci = tid (16 bytes) of each of the three tiles: of K and V, row
  // ci/16, slot ci%16; of K^T, row ci/4, slot ci%4; each wave's 64 chunks are contiguous.
  auto fetch = [&](int kb, DqTiles& T) {
    const int ci = tid, r = ci >> 4, x = (ci & 15) ^ (r & 15), d = ci >> 2, xt = (ci & 3) ^ ((d >> 2) & 3);
    const int lo = 16 * (64 * wave_u);
    gload_lds16(kd + (int64_t)(32 * kb + r) * 128 + 8 * x, reinterpret_cast<uint8_t*>(T.k) + lo);
    gload_lds16(vd + (int64_t)(32 * kb + r) * 128 + 8 * x, reinterpret_cast<uint8_t*>(T.v) + lo);
    gload_lds16(kdt + (int64_t)d * S + 32 * kb + 8 * xt, reinterpret_cast<uint8_t*>(T.kt) + lo);
  };
  // The K^T tile of "block -1" (the slot iteration 0 takes its dQ operands from) is zero: with zero dS
  // its products add exactly 0.
  {
    uint4* z = reinterpret_cast<uint4*>(buf[DQ_NBUF - 1].kt);
    z[tid] = uint4{0u, 0u, 0u, 0u};
  }
  fetch(0, buf[0]);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  uint32_t dsw[8] = {};  // dS^T of the previous block as bf16 pairs: slice t in dsw[4t .. 4t + 3]
  // dQ^T += K^T dS^T over a block's 32 keys, two 16-key steps: B slot (h, e) of step t is accumulator
  // element 8t + e, key 16t + 8(e/4) + 4h + e%4, the order (dq_tpos) of the K^T tile's rows
  auto kt_off = [&](int t, int dt) { return (32 * dt + c) * 32 + 8 * ((2 * t + h) ^ ((c >> 2) & 3)); };
  auto step = [&](auto kslot, int kb) {
    constexpr int s0 = decltype(kslot)::value;  // kb % 3
    // the next key block into the slot of block kb - 2, read last in iteration kb - 1
    if (kb + 1 < nkb) fetch(kb + 1, buf[(s0 + 1) % DQ_NBUF]);
    __builtin_amdgcn_sched_barrier(0);
    const DqTiles& T = buf[s0];
    const DqTiles& Tp = buf[(s0 + DQ_NBUF - 1) % DQ_NBUF];  // block kb - 1
    // S^T = K Q^T and dP^T = V dO^T: lane (query c, h), element i <-> key 8(i/4) + 4h + i%4 of the
    // block. The K and V operands of step s + 1 are read while the MFMAs of step s run, and the K^T
    // operands of block kb - 1 during the first four steps.
    auto off = [&](int s) { return c * 128 + 8 * ((2 * s + h) ^ (c & 15)); };  // columns 16s + 8h
    v8bf ka = ld8bf(T.k + off(0)), va = ld8bf(T.v + off(0));
    v8bf kta[2][4];
    v16f sacc, pacc;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      v8bf ka2, va2;
      if (s < 7) {
        ka2 = ld8bf(T.k + off(s + 1));
        va2 = ld8bf(T.v + off(s + 1));
      }
      if (s < 4) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int t = (2 * s + u) >> 2, dt = (2 * s + u) & 3;
          kta[t][dt] = ld8bf(Tp.kt + kt_off(t, dt));
        }
      }
      sacc = s == 0 ? mfma_bf16(ka, qop[0], v16f{}) : mfma_bf16(ka, qop[s], sacc);
      pacc = s == 0 ? mfma_bf16(va, gop[0], v16f{}) : mfma_bf16(va, gop[s], pacc);
      if (s < 7) {
        ka = ka2;
        va = va2;
      }
      if (s < 4) __builtin_amdgcn_sched_group_barrier(0x0100, 4, 0);
      else if (s < 7) __builtin_amdgcn_sched_group_barrier(0x0100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x0008, 2, 0);
    }
    // dQ^T products of block kb - 1, then P and dS of block kb on the VALU while they run
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const v8bf sb = __builtin_bit_cast(v8bf, uint4{dsw[4 * t], dsw[4 * t + 1], dsw[4 * t + 2], dsw[4 * t + 3]});
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) dqT[dt] = mfma_bf16(kta[t][dt], sb, dqT[dt]);
    }
    __builtin_amdgcn_sched_group_barrier(0x0008, 8, 0);
    float pv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) pv[i] = __builtin_amdgcn_exp2f(fmaf(sacc[i], P.scale_log2, -lse2));
    if (kb >= qb) {  // the block reaches this wave's queries: mask key > query
      const int qoff = 32 * (qb - kb);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + 4 * h + (i & 3) > qoff + c) pv[i] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)  // dS^T as bf16 pairs (elements 2e, 2e + 1)
      dsw[e] = pack_bf16(pv[2 * e] * (pacc[2 * e] - del), pv[2 * e + 1] * (pacc[2 * e + 1] - del));
    __builtin_amdgcn_sched_barrier(0);
    // The next key block's loads complete here; the barrier publishes them.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  };
  for (int kb = 0; kb < nkb; kb += 3) {
    step(std::integral_constant<int, 0>{}, kb);
    if (kb + 1 < nkb) step(std::integral_constant<int, 1>{}, kb + 1);
    if (kb + 2 < nkb) step(std::integral_constant<int, 2>{}, kb + 2);
  }
  {  // dQ^T products of the last block
    const DqTiles& Tp = buf[(nkb - 1) % DQ_NBUF];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const v8bf sb = __builtin_bit_cast(v8bf, uint4{dsw[4 * t], dsw[4 * t + 1], dsw[4 * t + 2], dsw[4 * t + 3]});
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) dqT[dt] = mfma_bf16(ld8bf(Tp.kt + kt_off(t, dt)), sb, dqT[dt]);
    }
  }
  if (!valid) return;
  const int64_t off = b * P.qsb + (int64_t)(q0 + c) * P.qss + hq * P.qsh + 4 * h;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      uint2 pq;
      pq.x = f32_to_bf16(dqT[dt][4 * g4] * P.scale) | (f32_to_bf16(dqT[dt][4 * g4 + 1] * P.scale) << 16);
      pq.y = f32_to_bf16(dqT[dt][4 * g4 + 2] * P.scale) | (f32_to_bf16(dqT[dt][4 * g4 + 3] * P.scale) << 16);
      *reinterpret_cast<uint2*>(P.dq + off + 32 * dt + 8 * g4) = pq;
    }
}

hipError_t launch_attn_bwd(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                           const uint8_t* vt, const uint8_t* vta, const uint16_t* o, const float* lse,
                           const uint16_t* dout, int B, int S, int Hq, int Hkv, float softmax_scale, int64_t qsb,
                           int64_t qss, int64_t qsh, int64_t ksb, int64_t kss, int64_t ksh, const BwdWorkspace& ws,
                           uint16_t* dq, uint16_t* dk, uint16_t* dv, hipStream_t stream) {
  const dim3 tq((unsigned)((S + 63) / 64), (unsigned)Hq, (unsigned)B), tk((unsigned)((S + 63) / 64), (unsigned)Hkv,
                                                                          (unsigned)B);
  bwd_prep_kernel<0, 1><<<tq, 256, 0, stream>>>(qc, qs, nullptr, 0, 0, 0, nullptr, 0, 0, 0, S, Hq, ws.qd, ws.qdt,
                                                   nullptr);
  bwd_prep_kernel<0, 1><<<tk, 256, 0, stream>>>(kc, ks, nullptr, 0, 0, 0, nullptr, 0, 0, 0, S, Hkv, ws.kd, ws.kdt, nullptr);
  bwd_prep_kernel<1><<<tk, 256, 0, stream>>>(vt, vta, nullptr, 0, 0, 0, nullptr, 0, 0, 0, S, Hkv, ws.vd, nullptr,
                                             nullptr);
  bwd_prep_kernel<2, 1><<<tq, 256, 0, stream>>>(nullptr, nullptr, dout, qsb, qss, qsh, o, qsb, qss, qsh, S, Hq,
                                                   ws.gd, ws.gdt, ws.delta, lse, ws.lse2);
  BwdParams p{};
  p.qd = ws.qd; p.qdt = ws.qdt; p.kd = ws.kd; p.kdt = ws.kdt; p.vd = ws.vd; p.gd = ws.gd; p.gdt = ws.gdt;
  p.lse = lse; p.delta = ws.delta; p.lse2 = ws.lse2;
  p.B = B; p.S = S; p.Hq = Hq; p.Hkv = Hkv;
  p.scale = softmax_scale;
  p.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.qsb = qsb; p.qss = qss; p.qsh = qsh; p.ksb = ksb; p.kss = kss; p.ksh = ksh;
  const unsigned tiles = (unsigned)((S + 127) / 128), dtiles = (unsigned)((S + 255) / 256);
  bwd_dkdv_kernel<<<dim3(tiles * (unsigned)Hkv * (unsigned)B), 256, 0, stream>>>(p);
  bwd_dq_kernel<<<dim3(dtiles * (unsigned)Hq * (unsigned)B), 512, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace mxfa
