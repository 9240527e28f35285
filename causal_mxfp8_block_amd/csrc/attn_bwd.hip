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
//  * dK/dV kernel: one wave per 16 keys, two waves per SIMD, their K and V operands held in registers
//    (16x16x32 MFMAs). For every query head of the KV head and every 32-query block at or after the
//    keys, it computes S = Q K^T and dP = dO V^T (keys on the lanes, queries on the accumulator
//    elements), P and dS elementwise, and accumulates dV^T += dO^T P and dK^T += Q^T dS. P and dS stay
//    in their accumulator registers and are the B operand of those MFMAs: the accumulator's query
//    order is a permutation of the B operand's contraction order, and the A operand (dO^T, Q^T, read
//    from LDS) is read in the same permuted order. The steps are software-pipelined.
//  * dQ kernel: one wave per 32 queries, their Q and dO operands in registers. For every 32-key block
//    at or before the queries it computes S^T = K Q^T and dP^T = V dO^T (queries on the lanes: lse and
//    Delta are per-lane scalars) and accumulates dQ^T += K^T dS^T the same way.
//  * Key > query is masked to P = 0. The loops start at the workgroup's first block on or below the
//    diagonal, so a wave whose own blocks start later computes at most three fully masked steps; that
//    keeps the loop branch-free per wave.
//  * Query (dK/dV) and key (dQ) blocks go from global memory straight into an LDS ring shared by the
//    workgroup (loads with the LDS flag, issued a step or two ahead; no register staging). Rows are
//    unpadded and the 16-byte chunks XOR-swizzled, so the operand reads are bank-conflict-free; the
//    preparation pass writes the transposed copies in each kernel's MFMA slot order.
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

// Position of query q (0..31) of a transposed dK/dV tile row: MFMA slot order, so that lane group g
// reads queries 4g..4g+3 and 16+4g..16+4g+3 as one 16-byte operand (positions 8g..8g+7).
__device__ __forceinline__ int dkdv_tpos(int q) { return 8 * ((q >> 2) & 3) + 4 * (q >> 4) + (q & 3); }
// Same for the dQ kernel's 32x32 operands: within each 16-token half, bits 2 and 3 swapped, so that lane
// half h reads tokens 4h..4h+3 and 8+4h..8+4h+3 of the half as one 16-byte operand.
__device__ __forceinline__ int dq_tpos(int q) { return (q & 16) | ((q & 4) << 1) | ((q & 8) >> 1) | (q & 3); }

// ---- preparation -------------------------------------------------------------------------------
// One workgroup per (b, h, 64-token tile), 256 threads: thread g handles token g/4, columns
// 32(g%4) .. +32. Source kSrc: 0 rowwise codes + E8M0 per 32 columns, 1 token-normalised codes + one
// E8M0 amplitude per token, 2 a bf16 [B,S,H,D] view (with Delta from the o view and lse * log2(e)
// from lse when delta != null). Writes the bf16 rows to out [B,H,S,D] and, when out_t != null, the
// transposed out_t [B,H,D,S]; with kSlot 1 (2) the tokens of each 32-token block of out_t are stored in
// the dK/dV (dQ) kernel's MFMA slot order, dkdv_tpos (dq_tpos), so that its tiles load as contiguous
// 16-byte pieces.
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
    const int pos = kSlot == 1 ? (dkdv_tpos(2 * e) >> 1) : kSlot == 2 ? (dq_tpos(2 * e) >> 1) : e;
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
  int S, Hq, Hkv;
  float scale, scale_log2;
  uint16_t *dq, *dk, *dv;                                // bf16 outputs (views)
  int64_t qsb, qss, qsh, ksb, kss, ksh;                 // strides of dq and of dk/dv
};

// ---- dK, dV ------------------------------------------------------------------------------------
// v_mfma_f32_16x16x32_bf16 (operand layout probed): A lane (m = l%16, g = l/16) element e <-> A[m][8g+e];
// B lane (n = l%16, g) element e <-> B[8g+e][n]; C lane (n = l%16, g) element i <-> C[4g+i][n].
typedef float v4f __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4f mfma16(const v8bf& a, const v8bf& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Global -> LDS without registers: lane l's 16 (or 4) bytes land at lds + 16 l (4 l); lds wave-uniform.
__device__ __forceinline__ void gload_lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)g, (__attribute__((address_space(3))) void*)lds,
                                   16, 0, 0);
}
__device__ __forceinline__ void gload_lds4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)g, (__attribute__((address_space(3))) void*)lds,
                                   4, 0, 0);
}

// Workgroup: 8 waves (two per SIMD) = keys 128 kt .. 128 kt + 127 of (b, hk); wave w owns keys
// 128 kt + 16 w + [0, 16), its K and V rows held in registers as B operands and its dK^T, dV^T
// accumulators (128 x 16 each) in registers. Steps n = (query head, 32-query block), the blocks from
// the last one down to 4kt: workgroups that run together read the same query block at the same time.
// Per step, keys on the MFMA columns: S = Q K^T and dP = dO V^T (two 16-query row tiles, K = D in four
// 32-wide steps), P and dS elementwise in the accumulators, then dV^T += dO^T P and dK^T += Q^T dS with
// P and dS as the B operand straight from those accumulators (element i of row tile mt is query
// 16mt + 4g + i: slot (g, e) of the contraction is query 16(e/4) + 4g + e%4, the order in which the
// preparation pass stores the transposed copies). Each step's tiles go from global memory straight
// into a ring of four LDS slots (loads with the LDS flag, no registers), two steps ahead. The loop is
// software-pipelined: while the VALU computes P and dS of step st, the matrix core runs the S and dP
// products of step st + 1 and the dV and dK products of step st - 1.
constexpr int DKDV_NBUF = 4;  // LDS ring: steps st - 1, st, st + 1 and st + 2 (arriving)
struct DkdvTiles {
  // Unpadded rows; reads stay conflict-free through XOR swizzles of the 16-byte chunks:
  uint16_t q[32 * 128], g[32 * 128];    // Q, dO rows: chunk c of row r in slot c ^ (r & 15)
  uint16_t qt[128 * 32], gt[128 * 32];  // Q^T, dO^T rows (slot order): chunk c of row d in slot c ^ ((d >> 2) & 3)
  float l[32], d[32];                   // lse * log2(e) and Delta of the step's 32 queries
};
// Step n_'s tiles from global memory straight into slot T (lane l's bytes at the wave's base + 16 l):
// thread tid fills LDS chunk tid (16 bytes) of each of the four tiles: of Q and dO, row r = tid/16,
// slot tid%16, holding chunk (tid%16) ^ (r & 15) of that query's row; of Q^T and dO^T, row d = tid/4,
// slot tid%4, holding chunk (tid%4) ^ ((d >> 2) & 3) of the block's 64 bytes of row d. Wave 0 also
// moves the 32 lse * log2(e) and 32 Delta values (4 bytes per lane).
__device__ __forceinline__ void dkdv_fetch(const uint16_t* __restrict__ qd, const uint16_t* __restrict__ gd,
                                           const uint16_t* __restrict__ qdt, const uint16_t* __restrict__ gdt,
                                           const float* __restrict__ lse2, const float* __restrict__ delta,
                                           DkdvTiles* __restrict__ T, int n_, int b, int hk, int G, int per_head,
                                           int nqb, int S, int Hq, int rr, int rx, int td, int tx, int lane,
                                           int wave_u) {
  const int hq_ = hk * G + n_ / per_head, q0_ = 32 * (nqb - 1 - n_ % per_head);
  const int64_t bhq_ = (int64_t)b * Hq + hq_;
  gload_lds16(qd + (bhq_ * S + q0_ + rr) * 128 + 8 * rx, reinterpret_cast<uint8_t*>(T->q) + 1024 * wave_u);
  gload_lds16(gd + (bhq_ * S + q0_ + rr) * 128 + 8 * rx, reinterpret_cast<uint8_t*>(T->g) + 1024 * wave_u);
  gload_lds16(qdt + (bhq_ * 128 + td) * S + q0_ + 8 * tx, reinterpret_cast<uint8_t*>(T->qt) + 1024 * wave_u);
  gload_lds16(gdt + (bhq_ * 128 + td) * S + q0_ + 8 * tx, reinterpret_cast<uint8_t*>(T->gt) + 1024 * wave_u);
  if (wave_u == 0) gload_lds4(lane < 32 ? lse2 + bhq_ * S + q0_ + lane : delta + bhq_ * S + q0_ + lane - 32, T->l);
}

// One iteration of the pipelined dK/dV loop: step st + 2's loads into slot L; the S and dP MFMAs of
// step st + 1 (tiles Tn, into sn, pn) and the dV and dK MFMAs of step st - 1 (tiles Tp, with its P
// and dS in pbp, sbp), one of each per group, interleaved with P and dS of step st (scores in sc, pc;
// lse and Delta from Tc). The slots and the global sources are restrict pointers: L is none of Tc,
// Tn, Tp, so the compiler can tell the LDS reads from the loads in flight and does not wait for
// those loads before the reads. Past the last step Tn is a stale slot (its products are unused).
__device__ __forceinline__ void dkdv_pipe_iter(
    const uint16_t* __restrict__ qd, const uint16_t* __restrict__ gd, const uint16_t* __restrict__ qdt,
    const uint16_t* __restrict__ gdt, const float* __restrict__ lse2, const float* __restrict__ delta,
    const DkdvTiles* __restrict__ Tc, const DkdvTiles* __restrict__ Tn, const DkdvTiles* __restrict__ Tp,
    DkdvTiles* __restrict__ L, int st, int nsteps, int b, int hk, int G, int per_head, int nqb, int S, int Hq, int rr,
    int rx, int td, int tx, int lane, int wave_u, int n, int g, int key0, float scale_log2, const v8bf (&kop)[4],
    const v8bf (&vop)[4], v4f (&dkT)[8], v4f (&dvT)[8], v4f (&sc)[2], v4f (&pc)[2], v4f (&sn)[2], v4f (&pn)[2],
    v8bf& pbp, v8bf& sbp) {
  if (st + 2 < nsteps)
    dkdv_fetch(qd, gd, qdt, gdt, lse2, delta, L, st + 2, b, hk, G, per_head, nqb, S, Hq, rr, rx, td, tx, lane, wave_u);
  const int qb = nqb - 1 - st % per_head;
  const int koff = key0 - 32 * qb;  // key - query offset of the two blocks' first tokens
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) sn[mt][i] = pn[mt][i] = 0.f;
  float lv[8], dv[8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const float4 l4 = *reinterpret_cast<const float4*>(Tc->l + 16 * mt + 4 * g);
    const float4 d4 = *reinterpret_cast<const float4*>(Tc->d + 16 * mt + 4 * g);
    lv[4 * mt] = l4.x; lv[4 * mt + 1] = l4.y; lv[4 * mt + 2] = l4.z; lv[4 * mt + 3] = l4.w;
    dv[4 * mt] = d4.x; dv[4 * mt + 1] = d4.y; dv[4 * mt + 2] = d4.z; dv[4 * mt + 3] = d4.w;
  }
  // operands of group k: rows 16(k/4) + n of Q and dO (step k%4 over D), row 16k + n of the transposes
  auto rowoff = [&](int k) { return (16 * (k >> 2) + n) * 128 + 8 * ((4 * (k & 3) + g) ^ n); };
  const int troff = n * 32 + 8 * (g ^ ((n >> 2) & 3));
  v8bf qa = ld8bf(Tn->q + rowoff(0)), ga = ld8bf(Tn->g + rowoff(0));
  v8bf gta = ld8bf(Tp->gt + troff), qta = ld8bf(Tp->qt + troff);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    v8bf qa2, ga2, gta2, qta2;
    if (k < 7) {  // the next group's operands, read one group ahead
      qa2 = ld8bf(Tn->q + rowoff(k + 1));
      ga2 = ld8bf(Tn->g + rowoff(k + 1));
      gta2 = ld8bf(Tp->gt + 16 * 32 * (k + 1) + troff);
      qta2 = ld8bf(Tp->qt + 16 * 32 * (k + 1) + troff);
    }
    const int mt = k >> 2, s4 = k & 3;
    sn[mt] = mfma16(qa, kop[s4], sn[mt]);
    pn[mt] = mfma16(ga, vop[s4], pn[mt]);
    dvT[k] = mfma16(gta, pbp, dvT[k]);
    dkT[k] = mfma16(qta, sbp, dkT[k]);
    {  // P and dS of element (mt, i) = (k/4, k%4) of step st; query 16mt + 4g + i, key key0 + n
      const int i = k & 3;
      float p = __builtin_amdgcn_exp2f(fmaf(sc[mt][i], scale_log2, -lv[k]));
      if (n + koff > 16 * mt + 4 * g + i) p = 0.f;  // key after query
      sc[mt][i] = p;
      pc[mt][i] = p * (pc[mt][i] - dv[k]);
    }
    if (k < 7) {
      qa = qa2; ga = ga2; gta = gta2; qta = qta2;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {  // slot (g, e) of the next dV/dK products: query 16(e/4) + 4g + e%4
    pbp[e] = (__bf16)sc[e >> 2][e & 3];
    sbp[e] = (__bf16)pc[e >> 2][e & 3];
  }
  // The loads issued at the top of this iteration (step st + 2) complete here; the barrier publishes them.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
}

__global__ __launch_bounds__(512, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkdv_kernel(const BwdParams P) {
  __shared__ __align__(16) DkdvTiles buf[DKDV_NBUF];
  const int S = P.S, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, g = lane >> 4;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int kt = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int G = P.Hq / P.Hkv;
  const int key0 = 128 * kt + 16 * wave;
  const bool valid = key0 < S;  // S % 32 == 0: a wave's 16 keys are all inside or all outside
  const int64_t bhk = (int64_t)b * P.Hkv + hk;
  // B operands: lane (key n, g), step s holds columns 32s + 8g + [0, 8) of the key's K and V rows.
  v8bf kop[4], vop[4];
  const int krow = valid ? key0 + n : 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    kop[s] = ld8bf(P.kd + (bhk * S + krow) * 128 + 32 * s + 8 * g);
    vop[s] = ld8bf(P.vd + (bhk * S + krow) * 128 + 32 * s + 8 * g);
  }
  v4f dkT[8], dvT[8];  // tile dt: lane (key n, g), element i <-> column d = 16dt + 4g + i
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) dkT[dt][i] = dvT[dt][i] = 0.f;
  const int nqb = S / 32, qb0 = 4 * kt, per_head = nqb - qb0, nsteps = G * per_head;
  // this thread's LDS chunk of the tiles (row and source chunk; the fetch below)
  const int rr = tid >> 4, rx = (tid & 15) ^ (rr & 15), td = tid >> 2, tx = (tid & 3) ^ ((td >> 2) & 3);
  // Slot 3 stands in for step -1 in iteration 0: zero transposed tiles, which with zero P and dS add
  // exactly 0. Step 3 first arrives there in iteration 1.
  {
    uint4* z0 = reinterpret_cast<uint4*>(buf[DKDV_NBUF - 1].qt);
    uint4* z1 = reinterpret_cast<uint4*>(buf[DKDV_NBUF - 1].gt);
    z0[tid] = uint4{0u, 0u, 0u, 0u};
    z1[tid] = uint4{0u, 0u, 0u, 0u};
  }
  dkdv_fetch(P.qd, P.gd, P.qdt, P.gdt, P.lse2, P.delta, &buf[0], 0, b, hk, G, per_head, nqb, S, P.Hq, rr, rx, td, tx,
             lane, wave_u);
  if (nsteps > 1)
    dkdv_fetch(P.qd, P.gd, P.qdt, P.gdt, P.lse2, P.delta, &buf[1], 1, b, hk, G, per_head, nqb, S, P.Hq, rr, rx, td, tx,
               lane, wave_u);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  // S and dP of step 0
  v4f sa[2], pa[2], sb[2], pb2[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sa[mt][i] = pa[mt][i] = 0.f;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int off = (16 * mt + n) * 128 + 8 * ((4 * s4 + g) ^ n);
      sa[mt] = mfma16(ld8bf(buf[0].q + off), kop[s4], sa[mt]);
      pa[mt] = mfma16(ld8bf(buf[0].g + off), vop[s4], pa[mt]);
    }
  }
  v8bf pbp, sbp;  // P and dS of the previous step (none before step 0)
#pragma unroll
  for (int e = 0; e < 8; ++e) pbp[e] = sbp[e] = (__bf16)0.f;
  // unrolled by four: ring slots are constants (step st in slot st % 4); S and dP buffers alternate
  auto it4 = [&](auto kslot, int st, v4f (&sc)[2], v4f (&pc)[2], v4f (&sn)[2], v4f (&pn)[2]) {
    constexpr int s = decltype(kslot)::value;
    dkdv_pipe_iter(P.qd, P.gd, P.qdt, P.gdt, P.lse2, P.delta, &buf[s], &buf[(s + 1) % DKDV_NBUF],
                   &buf[(s + 3) % DKDV_NBUF], &buf[(s + 2) % DKDV_NBUF], st, nsteps, b, hk, G, per_head, nqb, S, P.Hq,
                   rr, rx, td, tx, lane, wave_u, n, g, key0, P.scale_log2, kop, vop, dkT, dvT, sc, pc, sn, pn, pbp,
                   sbp);
  };
  for (int st = 0; st < nsteps; st += 4) {
    it4(std::integral_constant<int, 0>{}, st, sa, pa, sb, pb2);
    if (st + 1 < nsteps) it4(std::integral_constant<int, 1>{}, st + 1, sb, pb2, sa, pa);
    if (st + 2 < nsteps) it4(std::integral_constant<int, 2>{}, st + 2, sa, pa, sb, pb2);
    if (st + 3 < nsteps) it4(std::integral_constant<int, 3>{}, st + 3, sb, pb2, sa, pa);
  }
  {  // dV and dK of the last step
    const DkdvTiles& Tp = buf[(nsteps - 1) % DKDV_NBUF];
    const int troff = n * 32 + 8 * (g ^ ((n >> 2) & 3));
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      dvT[k] = mfma16(ld8bf(Tp.gt + 16 * 32 * k + troff), pbp, dvT[k]);
      dkT[k] = mfma16(ld8bf(Tp.qt + 16 * 32 * k + troff), sbp, dkT[k]);
    }
  }
  if (!valid) return;
  // lane (key n, g), element i of tile dt: column 16dt + 4g + i
  const int64_t off = b * P.ksb + (int64_t)(key0 + n) * P.kss + hk * P.ksh + 4 * g;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    uint2 pk, pv;
    pk.x = f32_to_bf16(dkT[dt][0] * P.scale) | (f32_to_bf16(dkT[dt][1] * P.scale) << 16);
    pk.y = f32_to_bf16(dkT[dt][2] * P.scale) | (f32_to_bf16(dkT[dt][3] * P.scale) << 16);
    pv.x = f32_to_bf16(dvT[dt][0]) | (f32_to_bf16(dvT[dt][1]) << 16);
    pv.y = f32_to_bf16(dvT[dt][2]) | (f32_to_bf16(dvT[dt][3]) << 16);
    *reinterpret_cast<uint2*>(P.dk + off + 16 * dt) = pk;
    *reinterpret_cast<uint2*>(P.dv + off + 16 * dt) = pv;
  }
}

// ---- dQ ----------------------------------------------------------------------------------------
// Workgroup: 4 waves = queries 128 qt .. 128 qt + 127 of (b, hq); wave w owns queries 32(4qt + w) + [0, 32).
// Key blocks go from global memory straight into two LDS slots (loads with the LDS flag), one step
// ahead, as in the dK/dV kernel.
struct DqTiles {
  uint16_t k[32 * 128], v[32 * 128];  // K, V rows: chunk c of row r in slot c ^ (r & 15)
  uint16_t kt[128 * 32];              // K^T rows (dQ slot order): chunk c of row d in slot c ^ ((d >> 2) & 3)
};
__global__ __launch_bounds__(256, 2) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(const BwdParams P) {
  __shared__ __align__(16) DqTiles buf[2];
  const int S = P.S, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 31, h = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int qt = blockIdx.x, hq = blockIdx.y, b = blockIdx.z;
  const int hk = hq / (P.Hq / P.Hkv);
  const int qb = 4 * qt + wave, q0 = 32 * qb;
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
  const int nkb = min(4 * qt + 3, S / 32 - 1) + 1;  // key blocks any wave of the workgroup needs
  // Thread tid fills LDS chunks ci = tid + 256 i (i = 0, 1; 16 bytes each) of the three tiles: of K and
  // V, row ci/16, slot ci%16; of K^T, row ci/4, slot ci%4; each wave's 64 chunks are contiguous.
  auto fetch = [&](int kb, DqTiles& T) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ci = tid + 256 * i, r = ci >> 4, x = (ci & 15) ^ (r & 15), d = ci >> 2, xt = (ci & 3) ^ ((d >> 2) & 3);
      const int lo = 16 * (256 * i + 64 * wave_u);
      gload_lds16(kd + (int64_t)(32 * kb + r) * 128 + 8 * x, reinterpret_cast<uint8_t*>(T.k) + lo);
      gload_lds16(vd + (int64_t)(32 * kb + r) * 128 + 8 * x, reinterpret_cast<uint8_t*>(T.v) + lo);
      gload_lds16(kdt + (int64_t)d * S + 32 * kb + 8 * xt, reinterpret_cast<uint8_t*>(T.kt) + lo);
    }
  };
  fetch(0, buf[0]);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    // the next key block into the other slot, read last in step kb - 1 (before the barrier ending it)
    if (kb + 1 < nkb) fetch(kb + 1, buf[(kb + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
    const DqTiles& T = buf[kb & 1];
    {  // branch-free as in the dK/dV kernel
      // S^T = K Q^T and dP^T = V dO^T: lane (query c, h), element i <-> key 8(i/4) + 4h + i%4 of the block
      v8bf ka[8], va[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int off = c * 128 + 8 * ((2 * s + h) ^ (c & 15));  // columns 16s + 8h: chunk 2s + h
        ka[s] = ld8bf(T.k + off);
        va[s] = ld8bf(T.v + off);
      }
      v16f sacc, pacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = pacc[i] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        sacc = mfma_bf16(ka[s], qop[s], sacc);
        pacc = mfma_bf16(va[s], gop[s], pacc);
      }
      v8bf kta[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)  // row 32dt + c, chunk 2t + h
          kta[t][dt] = ld8bf(T.kt + (32 * dt + c) * 32 + 8 * ((2 * t + h) ^ ((c >> 2) & 3)));
      const int qoff = 32 * (qb - kb);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = 8 * (i >> 2) + 4 * h + (i & 3);
        float p = __builtin_amdgcn_exp2f(fmaf(sacc[i], P.scale_log2, -lse2));
        if (kk > qoff + c) p = 0.f;  // key after query (whole block when kb > qb)
        pacc[i] = p * (pacc[i] - del);  // dS^T
      }
      // dQ^T += K^T dS^T over the 32 keys, two 16-key steps: B slot (h, e) of step t is accumulator
      // element 8t + e, key 16t + 8(e/4) + 4h + e%4, the order (dq_tpos) of the K^T tile's rows
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const v8bf sb = to_bf16(pacc, t);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) dqT[dt] = mfma_bf16(kta[t][dt], sb, dqT[dt]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // The next key block's loads complete here; the barrier publishes them.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
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
  bwd_prep_kernel<0, 2><<<tk, 256, 0, stream>>>(kc, ks, nullptr, 0, 0, 0, nullptr, 0, 0, 0, S, Hkv, ws.kd, ws.kdt, nullptr);
  bwd_prep_kernel<1><<<tk, 256, 0, stream>>>(vt, vta, nullptr, 0, 0, 0, nullptr, 0, 0, 0, S, Hkv, ws.vd, nullptr,
                                             nullptr);
  bwd_prep_kernel<2, 1><<<tq, 256, 0, stream>>>(nullptr, nullptr, dout, qsb, qss, qsh, o, qsb, qss, qsh, S, Hq,
                                                   ws.gd, ws.gdt, ws.delta, lse, ws.lse2);
  BwdParams p{};
  p.qd = ws.qd; p.qdt = ws.qdt; p.kd = ws.kd; p.kdt = ws.kdt; p.vd = ws.vd; p.gd = ws.gd; p.gdt = ws.gdt;
  p.lse = lse; p.delta = ws.delta; p.lse2 = ws.lse2;
  p.S = S; p.Hq = Hq; p.Hkv = Hkv;
  p.scale = softmax_scale;
  p.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.qsb = qsb; p.qss = qss; p.qsh = qsh; p.ksb = ksb; p.kss = kss; p.ksh = ksh;
  const unsigned tiles = (unsigned)((S + 127) / 128);
  bwd_dkdv_kernel<<<dim3(tiles, (unsigned)Hkv, (unsigned)B), 512, 0, stream>>>(p);
  bwd_dq_kernel<<<dim3(tiles, (unsigned)Hq, (unsigned)B), 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace mxfa
