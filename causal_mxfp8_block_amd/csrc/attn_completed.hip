// attn_completed.hip -- completed-block partial of leak-free causal MXFP8 attention, gfx950.
//
// TransformerEngine PR #3865, "Description", first bullet: query i attends in MXFP8 to every key of
// the 32-token blocks that end at or before its own block, j < 32*floor(i/32); every columnwise V
// scale read there covers visible tokens only. This is nearly all of the attention FLOPs.
//
// Design (CDNA4, wave64):
//  * A workgroup is 4 waves; wave w owns the 32 queries of one 32-token block, so its key range is
//    [0, 32*cb) with no per-element mask: the completed-block mask is block-granular.
//  * Scores are computed transposed, S^T = K . Q^T, with the block-scaled FP8 MFMA
//    v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 operands, one E8M0 per 32 along D on both sides). The
//    accumulator then holds one query per lane (lane & 31) and 16 keys per 32-key block, so row
//    statistics are lane-local up to one exchange with lane ^ 32 (v_permlane32_swap).
//  * The K rows of each 32-key block sit in LDS in a permuted order chosen so that accumulator
//    element i of lane (c, hf) is key 16hf + i: exactly the bytes lane (c, hf) must supply as the
//    B operand of O^T = V^T . P^T. The E4M3 codes of P therefore go into that MFMA where they were
//    computed, with no cross-lane traffic.
//  * Online softmax in the log2 domain with an integer running exponent T: p = 2^(t - T). T is
//    raised only when a block maximum of p would exceed 224 (lazy rescale); the E8M0 quantisation of
//    P commutes with powers of two, so the P codes do not depend on T.
//  * The E8M0 exponent of each (query, 32-key block) of P comes from the block maximum taken on the
//    raw scores: the fma that forms t is monotone, so k = ceil(scale * max s - T - log2 448), one fma
//    with -(T + log2 448) kept per lane, is the smallest k with max p <= 448 * 2^k. Lane half hf
//    computes it for block hf, whose byte it supplies as the P.V scale operand, and one exchange
//    gives every lane both. The exponent is then folded into the exponential, p / 2^k =
//    2^(t - T - k), so the plain v_cvt_pk_fp8_f32 gives the E4M3 codes; the normaliser sums p / 2^k
//    per block and rescales the two block sums by 2^k. P.V is the block-scaled FP8 MFMA again, on
//    the columnwise V codes (keys contiguous per column).
//  * O^T leaves one query per lane too, so the rescale and the final 1/l are per-lane scalars.
//  * K and V tiles of 64 keys go from HBM straight into LDS (buffer loads with the LDS flag), once per
//    workgroup, shared by the 4 waves: double-buffered, one barrier per tile. No register holds a
//    tile in flight. A tile's loads are issued after the score MFMAs of the previous tile, so the
//    wait for them falls after that tile's softmax.
//  * Three workgroups per CU (three waves per SIMD, at most 168 VGPRs each): one wave's softmax VALU
//    work overlaps the MFMAs, LDS reads and barrier waits of the other two. Within a wave the loop is
//    plain (scores, softmax, P.V), with the V operands read next to their MFMAs so that few
//    registers live across the softmax; a software-pipelined loop that overlaps MFMA and VALU within
//    one wave needs 255 VGPRs, allows only two waves per SIMD, and is slower.
//  * Full tiles and the half tile at the end of a wave's range are separate code paths, so the
//    common path has no per-element select.
//  * One-dimensional grid in global longest-first order: all (batch, head) pairs of the last query
//    tile, then of the one before, and so on (the causal work of a query tile grows with its
//    index), so the machine drains evenly. Consecutive workgroup ids go to different XCDs in turn;
//    the pair index is permuted so that the workgroups one XCD receives are adjacent (batch, head)
//    pairs, i.e. query heads that share a KV head under GQA, which share K/V in that XCD's L2.
#include "device_common.h"
#include "launch.h"

#include <type_traits>

namespace mxfa {

constexpr int CB_BM = 128;    // queries per workgroup (4 waves x 32)
constexpr int CB_BN = 64;     // keys per tile (two 32-key MX blocks)
// K and V tiles go from HBM straight into LDS (buffer loads with the LDS flag: each lane's 16 bytes
// land at consecutive LDS addresses), so their rows are unpadded. Reads stay conflict-free through an
// XOR swizzle of the 16-byte chunks: chunk x of K row r sits in slot x ^ ((r >> 1) & 7), chunk x of V
// column d in slot x ^ ((d >> 2) & 3).
constexpr int CB_KROW = 128;  // LDS bytes per K row
constexpr int CB_VROW = 64;   // LDS bytes per V column (keys contiguous)
constexpr float CB_LOG2_448 = 8.80735492205760410f;  // log2 of the largest E4M3 value
constexpr int CB_RSRC_W3 = 0x00020000;  // buffer descriptor word 3 on gfx9: 32-bit data, raw offsets

struct __align__(16) TileSmem {
  uint8_t k[CB_BN * CB_KROW];  // K codes, key-major
  uint8_t v[128 * CB_VROW];    // V codes, column-major (keys contiguous)
  uint32_t ks[CB_BN];          // the 4 E8M0 bytes of each key, stored in the byte order s0 s2 s1 s3
  uint8_t vs[2 * 128];         // E8M0 bytes of the two key blocks: [block][c][dt] for column 32dt + c
};

__device__ __forceinline__ v8i make_v8i(uint4 a, uint4 b) {
  v8i r;
  r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
  r[4] = (int)b.x; r[5] = (int)b.y; r[6] = (int)b.z; r[7] = (int)b.w;
  return r;
}

// IEEE 754-2019 maximum (v_maximum3_f32 on gfx950): unlike fmaxf it needs no NaN quieting of
// MFMA results first. Every input here is finite.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// A VGPR whose previous contents do not matter: the empty asm defines it without an instruction, so
// packing four codes does not first clear the half-word the second conversion fills.
__device__ __forceinline__ int fresh_reg() {
  int u;
  asm volatile("" : "=v"(u));
  return u;
}

// E4M3 codes of four fp32 values (round to nearest even; every value here is at most 464, which
// converts to 448), a in the lowest byte.
__device__ __forceinline__ int pack4_p(float a, float b, float c, float d) {
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, fresh_reg(), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Block-scaled FP8 MFMA whose A and B scales are byte kSelA / kSelB of the scale registers.
template <int kSelA, int kSelB>
__device__ __forceinline__ v16f mfma_mx(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, kSelA, sa, kSelB, sb);
}

// Exchange with lane ^ 32 (v_permlane32_swap): afterwards x holds, in lanes 32..63, what y held in
// lanes 0..31, and y holds, in lanes 0..31, what x held in lanes 32..63.
__device__ __forceinline__ void swap32(uint32_t& x, uint32_t& y) {
  auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  x = r[0];
  y = r[1];
}
__device__ __forceinline__ void swap32f(float& x, float& y) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = __builtin_bit_cast(uint32_t, y);
  swap32(a, b);
  x = __builtin_bit_cast(float, a);
  y = __builtin_bit_cast(float, b);
}

// One thread's share of a tile load, through buffer resources over the current (b, kv-head) slice,
// straight into LDS: thread tid fills LDS chunks c = 256 i + tid (i = 0, 1) of the K tile (row c/8,
// slot c%8, from byte offset kvoff) and of the V tile (column c/4, slot c%4, from byte offset vvoff);
// the wave's 64 chunks of one instruction are contiguous. In waves 0 and 1 it also loads one scale
// word into sc: wave 0 the 4 E8M0 bytes of key tid, wave 1 one word of the tile's two V scale blocks.
// The per-tile offset is a scalar.
#define TILE_LOAD(T, sc, kt0)                                                                    \
  do {                                                                                           \
    bload_lds16(rk, (T).k + 16 * (64 * wave_u), kvoff0, (kt0) * 128);                            \
    bload_lds16(rk, (T).k + 16 * (256 + 64 * wave_u), kvoff1, (kt0) * 128);                      \
    bload_lds16(rv, (T).v + 16 * (64 * wave_u), vvoff0, (kt0));                                  \
    bload_lds16(rv, (T).v + 16 * (256 + 64 * wave_u), vvoff1, (kt0));                            \
    if (wave_u < 2)                                                                              \
      sc = __builtin_amdgcn_raw_buffer_load_b32(rs, svoff, wave_u == 0 ? (kt0) * 4 : ((kt0) >> 5) * 128, 0); \
  } while (0)

__device__ __forceinline__ int k_lds_row(int kk) {
  return (kk & 32) | (((kk >> 2) & 3) << 3) | (((kk >> 4) & 1) << 2) | (kk & 3);
}
__device__ __forceinline__ int k_row_key(int r) {  // inverse of k_lds_row: the key stored in LDS row r
  return (r & 32) | (((r >> 3) & 3) << 2) | (((r >> 2) & 1) << 4) | (r & 3);
}
__device__ __forceinline__ int k_slot(int r, int x) { return x ^ ((r >> 1) & 7); }
__device__ __forceinline__ int v_slot(int d, int x) { return x ^ ((d >> 2) & 3); }
// 16 bytes per lane from a buffer resource straight into LDS: lane l's bytes go to lds + 16 l.
__device__ __forceinline__ void bload_lds16(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// kFresh: the slot addresses are formed here from an opaque copy of tid (the ordinary causal variant,
// which has no register to keep them in across its loop).
template <bool kFresh>
__device__ __forceinline__ void store_scales(TileSmem& t, uint32_t sc, int tid) {
  if (kFresh) asm volatile("" : "+v"(tid));
  if (tid < 64) {
    // bytes s0 s2 s1 s3: the 16-bit half hf then holds the scales of D-blocks hf and 2 + hf
    t.ks[k_lds_row(tid)] = __builtin_amdgcn_perm(sc, sc, 0x03010200u);
  } else if (tid < 128) {
    // the word holds columns d = 4w .. 4w+3 of block w / 32 (w = tid - 64); store column d = 32dt + c
    // at [block][c][dt] so that one dword read gives a lane its four d-tiles' scales
    const int w = tid - 64, blk = w >> 5, d0 = (w & 31) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int dd = d0 + e;
      t.vs[blk * 128 + (dd & 31) * 4 + (dd >> 5)] = (uint8_t)(sc >> (8 * e));
    }
  }
}

// Per-wave running state of the online softmax.
struct RowState {
  v16f o[4];   // O^T accumulator: lane (c, hf), element i of tile dt -> column 32dt + 8(i/4) + 4hf + i%4
  float nT;    // -T: the integer-valued running exponent T, negated (set on the wave's first tile)
  float nTL;   // -(T + log2 448)
  float lsum;  // this lane's share of sum p
};

// S^T = K Q^T for one 64-key tile (kFull) or its first 32-key block only. Lane (c, hf), element i of
// sacc[kt] is the score of query c against key 32kt + 16hf + i (the K rows are permuted in LDS).
// kFresh (the ordinary causal variant): on the half-tile path the lane's scale offset is formed afresh
// from an opaque copy, which spares that variant its register spills (2% faster there). The leak-free
// kernels keep the offset computed once, spilled to 4 bytes of scratch that only the half tile and the
// first tile reload: forming it afresh there is 1% slower.
template <bool kFull, bool kFresh = false>
__device__ __forceinline__ void scores(v16f (&sacc)[2], const TileSmem& t, const v8i (&qop)[2], const int (&qsc)[2],
                                       int c, int hf) {
  constexpr int nkt = kFull ? 2 : 1;
  // All K operands first, so the LDS round trips overlap. Lane (c, hf) supplies row c of each 32-key
  // block: bytes d = 64m + 16hf + [0,16) and 64m + 32 + 16hf + [0,16); its scale for step m is byte m
  // of the 16-bit half hf of the row's permuted scale word.
  v8i kop[nkt][2];
  int ksc[nkt];
#pragma unroll
  for (int kt = 0; kt < nkt; ++kt) {
    const int r = 32 * kt + c;
    const uint8_t* kr = t.k + r * CB_KROW;
#pragma unroll
    for (int m = 0; m < 2; ++m)
      kop[kt][m] = make_v8i(*reinterpret_cast<const uint4*>(kr + 16 * k_slot(r, 4 * m + hf)),
                            *reinterpret_cast<const uint4*>(kr + 16 * k_slot(r, 4 * m + 2 + hf)));
    if (kFresh && !kFull) {
      int so = 4 * c + 2 * hf;  // this lane's scale offset
      asm volatile("" : "+v"(so));
      ksc[kt] = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(t.ks) + 128 * kt + so);
    } else {
      ksc[kt] = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(t.ks) + (32 * kt + c) * 4 + 2 * hf);
    }
  }
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[kt][i] = 0.f;
  // Independent accumulators alternate, so no MFMA waits on the one just issued.
#pragma unroll
  for (int kt = 0; kt < nkt; ++kt) sacc[kt] = mfma_mx<0, 0>(kop[kt][0], qop[0], sacc[kt], ksc[kt], qsc[0]);
#pragma unroll
  for (int kt = 0; kt < nkt; ++kt) sacc[kt] = mfma_mx<1, 0>(kop[kt][1], qop[1], sacc[kt], ksc[kt], qsc[1]);
}

// Softmax, P quantisation and O^T += V^T P^T for one tile whose scores are in sacc. kFull: both 32-key
// blocks are visible keys of this wave; otherwise only the first one is (the second one's p is zero).
// kMaskBlk (ordinary causal variant only): that block is the wave's own 32-token block, of which query
// qw + c sees keys qw .. qw + c; the others get p = 0, and its E8M0 comes from the visible keys. The V
// operands are read from LDS just before their MFMAs, at the end: the fewest registers live across
// the softmax, which lets three waves share a SIMD.
template <bool kFull, int kMaskBlk = -1>
__device__ __forceinline__ void softmax_pv(RowState& st, v16f (&sacc)[2], const TileSmem& t, float scale_log2, int c,
                                           int hf, bool first) {
  // Lane (c, hf), element i of block kt holds key 32kt + 16hf + i of the tile, query c.
  if (kMaskBlk >= 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (16 * hf + i > c) sacc[kMaskBlk][i] = -INFINITY;
  }
  float m0 = sacc[0][0], m1 = kFull ? sacc[1][0] : -INFINITY;
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    m0 = vmax(m0, sacc[0][i]);
    if (kFull) m1 = vmax(m1, sacc[1][i]);
  }
  // After the exchange lane half hf holds both halves of block hf's maximum (its own block: the one
  // whose E8M0 byte it supplies as the P.V scale operand).
  swap32f(m0, m1);
  const float Mown = vmax(m0, m1);
  // E8M0 exponent of the own block of P: the smallest k with max p <= 448 * 2^k, with p = 2^(t - T)
  // and the fma that forms t monotone, k = ceil(scale_log2 * max s - T - log2 448), clamped at
  // -127 as the scale rule clamps it (byte 0). An empty block (-inf) gets -127.
  float kown = vmax(ceilf(fmaf(Mown, scale_log2, st.nTL)), -127.f);
  // Raise T when a block maximum of p would exceed 224 (k >= 0): lazy rescale by an exact power of
  // two. After the first tile T only rises: a query whose maximum lies below its T keeps it, so its
  // accumulator and sum are never scaled up (a large upward scale could overflow).
  if (first || __any(kown >= 0.f)) {
    float x0 = fmaf(Mown, scale_log2, st.nT), x1 = x0;  // log2 of each block's largest p
    swap32f(x0, x1);
    const float up = ceilf(vmax(x0, x1));
    const float shift = first ? up : vmax(up, 0.f);
    const float f = first ? 0.f : __builtin_amdgcn_exp2f(-shift);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.o[dt][i] *= f;
    st.lsum *= f;
    st.nT -= shift;
    st.nTL -= shift;
    kown = vmax(ceilf(fmaf(Mown, scale_log2, st.nTL)), -127.f);
  }
  // The own block's byte is the P.V B-operand scale of this lane half; both exponents in every lane
  // (k0, k1) for the elements: nb = -T - k folds the exponent into the exponential.
  const int psc = (int)kown + 127;
  float k0 = kown, k1 = kown;
  swap32f(k0, k1);
  const float nb0 = st.nT - k0, nb1 = st.nT - k1;

  v8i pop;
  float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float q[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) q[e] = __builtin_amdgcn_exp2f(fmaf(sacc[0][4 * g + e], scale_log2, nb0));
    {
      const float s4 = (q[0] + q[1]) + (q[2] + q[3]);
      ls0 = g == 0 ? s4 : ls0 + s4;  // no add of the initial zero
    }
    pop[g] = pack4_p(q[0], q[1], q[2], q[3]);
    if (kFull) {
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = __builtin_amdgcn_exp2f(fmaf(sacc[1][4 * g + e], scale_log2, nb1));
      const float s4 = (q[0] + q[1]) + (q[2] + q[3]);
      ls1 = g == 0 ? s4 : ls1 + s4;
      pop[4 + g] = pack4_p(q[0], q[1], q[2], q[3]);
    } else {
      pop[4 + g] = 0;
    }
  }
  st.lsum += kFull ? ldexpf(ls0, (int)k0) + ldexpf(ls1, (int)k1) : ldexpf(ls0, (int)k0);
  // This tile's V^T operand of d-tile dt: lane (c, hf) supplies column 32dt + c, keys 16hf + [0,16) and
  // 32 + 16hf + [0,16); its scales are byte dt of the word of column c.
  const uint32_t vsw = *reinterpret_cast<const uint32_t*>(t.vs + hf * 128 + c * 4);
  auto vop = [&](int dt) {
    const int d = 32 * dt + c;
    const uint8_t* vr = t.v + d * CB_VROW;
    return make_v8i(*reinterpret_cast<const uint4*>(vr + 16 * v_slot(d, hf)),
                    *reinterpret_cast<const uint4*>(vr + 16 * v_slot(d, 2 + hf)));
  };
  // All four V operands are read before the first P.V MFMA (the score registers are free by now), so
  // the LDS latency is paid once rather than before each MFMA.
  const v8i v0 = vop(0), v1 = vop(1), v2 = vop(2), v3 = vop(3);
  __builtin_amdgcn_sched_group_barrier(0x0100, 9, 0);  // the 8 operand reads and the scale word
  __builtin_amdgcn_sched_group_barrier(0x0008, 4, 0);  // then the 4 MFMAs
  st.o[0] = mfma_mx<0, 0>(v0, pop, st.o[0], (int)vsw, psc);
  st.o[1] = mfma_mx<1, 0>(v1, pop, st.o[1], (int)vsw, psc);
  st.o[2] = mfma_mx<2, 0>(v2, pop, st.o[2], (int)vsw, psc);
  st.o[3] = mfma_mx<3, 0>(v3, pop, st.o[3], (int)vsw, psc);
}

struct AttnParams {
  const uint8_t *qc, *qs, *kc, *ks, *vc, *vcs;  // rowwise Q/K and columnwise V codes/scales
  const uint8_t *vt, *vta;                       // token-normalised V (fused epilogue only)
  const uint16_t* qbf;                           // fused only: bf16 Q view quantised in-kernel (else qc/qs)
  int64_t qsb, qss, qsh;                         // ... its element strides
  int S, Hq, Hkv, n_qtiles;
  int n_pairs;                                   // B * Hq
  int xcd_pairs;                                 // n_pairs / 8 when n_pairs % 8 == 0, else 0
  float scale_log2;                              // softmax_scale * log2(e)
  float *o_c, *lse_c;                            // completed partial (unfused)
  void* out;                                     // final output view (fused)
  int64_t osb, oss, osh;
  int out_bf16;
  int out_mxfp8;                                 // fused: O as E4M3 codes + one E8M0 per 32 columns
  uint8_t* sf_o;                                 // ... those E8M0 bytes, [B,Hq,S,D/32]
  float* lse_out;                                // may be null (fused)
};

// LDS: the double-buffered K/V tiles of the main loop, reused afterwards (fused epilogue) for each
// wave's decoded token-normalised own-block V, 32 keys x 128 columns of bf16 (exact: E4M3 values times
// a power of two need 4 significant bits).
constexpr int CB_NBUF = 2;  // this tile, the next one arriving
constexpr int CB_LDS_BYTES = CB_NBUF * sizeof(TileSmem);
static_assert(4 * 32 * 128 * 2 <= CB_LDS_BYTES, "the own-block V must fit the tile buffers");

// kMode: MODE_COMPLETED, the completed-block partial (O_c, lse_c); MODE_FUSED, the whole attention of
// the row: completed blocks, the own block on the token-normalised V (TE#3865 Description, second
// bullet), and the merge through the log-sum-exps, written once in the output's layout;
// MODE_LEAKY, ordinary causal MXFP8 (keys j <= i, the own block through the same MXFP8 P.V with
// its columnwise V scales, which also cover later tokens: the variant TE#3865 replaces, its
// "MXFP8" column under Performance), written in the output's layout.
enum : int { MODE_COMPLETED = 0, MODE_FUSED = 1, MODE_LEAKY = 2 };
template <int kMode>
__global__ __launch_bounds__(256, 3) void attn_kernel(const AttnParams P) {
  constexpr bool kFused = kMode == MODE_FUSED, kLeaky = kMode == MODE_LEAKY;
  __shared__ __align__(16) uint8_t lds[CB_LDS_BYTES];
  TileSmem* sm = reinterpret_cast<TileSmem*>(lds);  // sm[0], sm[1]
  const int S = P.S;
  const uint8_t *__restrict__ kc = P.kc, *__restrict__ ks = P.ks, *__restrict__ vc = P.vc,
                *__restrict__ vcs = P.vcs;
  const float scale_log2 = P.scale_log2;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // the same, as a scalar (tile loads only)
  const int c = lane & 31, hf = lane >> 5;
  // Workgroup id -> (query tile, pair): round r = id / n_pairs takes query tile n_qtiles - 1 - r; the
  // pair index within the round is permuted so that the ids one XCD receives (id mod 8 equal) cover
  // n_pairs / 8 adjacent pairs.
  const int id = (int)blockIdx.x;
  const int round = id / P.n_pairs, slot = id - round * P.n_pairs;
  const int qtile = P.n_qtiles - 1 - round;
  const int pair = P.xcd_pairs ? (slot & 7) * P.xcd_pairs + (slot >> 3) : slot;
  const int b = pair / P.Hq, hq = pair - b * P.Hq;
  const int hk = hq / (P.Hq / P.Hkv);
  const int q0 = qtile * CB_BM;
  const int qw = q0 + 32 * wave;          // first query of this wave; its completed keys are j < qw
  const bool wave_valid = qw < S;
  const int e_w = wave_valid ? qw : 0;
  const int e_wg = min(q0 + 96, S - 32);  // completed-key range end of the last valid wave
  // (the ordinary causal variant also reads the last wave's own block)
  const int ntiles = (e_wg + (kLeaky ? 32 : 0) + CB_BN - 1) / CB_BN;
  const int64_t bhq = (int64_t)b * P.Hq + hq, bhk = (int64_t)b * P.Hkv + hk;
  // Buffer resources over this kv head's K codes [S,128], V codes [128,S] and K or V scales. The
  // record count is an unsigned 32-bit field: S <= 2^24 (checked on the host) keeps S * 128 <= 2^31
  // and every per-lane and per-tile offset below it within a signed 32-bit int.
  const int nrec_codes = (int)((uint32_t)S * 128u), nrec_scales = (int)((uint32_t)S * 4u);
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kc + bhk * S * 128), 0, nrec_codes, CB_RSRC_W3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vc + bhk * S * 128), 0, nrec_codes, CB_RSRC_W3);
  const __amdgpu_buffer_rsrc_t rs =
      wave_u == 0
          ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(ks + bhk * S * 4), 0, nrec_scales, CB_RSRC_W3)
          : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vcs + bhk * S * 4), 0, nrec_scales, CB_RSRC_W3);
  // Per-lane source offsets of the tile loads (the tile's own offset is a scalar): LDS chunk c of K is
  // row r = c/8 (key k_row_key(r)), slot c%8, holding chunk k_slot(r, c%8); of V, column c/4, slot c%4.
  int kvoff0, kvoff1, vvoff0, vvoff1;
  {
    const int c0 = tid, c1 = tid + 256;
    kvoff0 = k_row_key(c0 >> 3) * 128 + 16 * k_slot(c0 >> 3, c0 & 7);
    kvoff1 = k_row_key(c1 >> 3) * 128 + 16 * k_slot(c1 >> 3, c1 & 7);
    vvoff0 = (c0 >> 2) * S + 16 * v_slot(c0 >> 2, c0 & 3);
    vvoff1 = (c1 >> 2) * S + 16 * v_slot(c1 >> 2, c1 & 3);
  }
  const int svoff = (tid & 63) * 4;

  // Q^T operand (B of S^T = K Q^T) for the two 64-wide K steps over D. Lane (c, hf) holds bytes
  // d = 64m + 16hf + [0,16) and 64m + 32 + 16hf + [0,16) of query qw + c; its scale is that of
  // D-block 2m + hf.
  v8i qop[2] = {};
  int qsc[2] = {127, 127};
  if (kFused && P.qbf) {
    // Q quantised here from bf16, with the rowwise quantiser's rule (TE#3865 Description: Q in MXFP8
    // with one E8M0 per 32 elements of D): lane (c, hf) holds, for step m, halves of D-blocks 2m
    // (d = 64m + 16hf + [0,16)) and 2m + 1 (d = 64m + 32 + 16hf + [0,16)); the other halves are in lane
    // c + 32(1 - hf), whose maxima complete the block amax. Same operations as the quantiser, so the
    // codes and scales are identical to its output.
    const int row = wave_valid ? qw + c : 0;
    const uint16_t* xrow = P.qbf + b * P.qsb + (int64_t)row * P.qss + hq * P.qsh;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float v[2][16];
      float am[2];
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        const uint4* src = reinterpret_cast<const uint4*>(xrow + 64 * m + 32 * part + 16 * hf);
        const uint4 r0 = src[0], r1 = src[1];
        const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          v[part][2 * i] = bf16_to_f32(w[i] & 0xffffu);
          v[part][2 * i + 1] = bf16_to_f32(w[i] >> 16);
          a = fmaxf(a, fabsf(v[part][2 * i]));
          a = fmaxf(a, fabsf(v[part][2 * i + 1]));
        }
        am[part] = fmaxf(a, __shfl_xor(a, 32));
      }
      uint32_t cw[8];
      int kb[2];
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        kb[part] = e8m0_exponent(am[part]);
        const float f = pow2_neg(kb[part]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          cw[4 * part + j] = pack4_e4m3(v[part][4 * j] * f, v[part][4 * j + 1] * f, v[part][4 * j + 2] * f,
                                        v[part][4 * j + 3] * f);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) qop[m][j] = (int)cw[j];
      qsc[m] = (hf ? kb[1] : kb[0]) + 127;
    }
  } else if (wave_valid) {
    const uint8_t* qrow = P.qc + (bhq * S + qw + c) * 128;
    const uint32_t sw = *reinterpret_cast<const uint32_t*>(P.qs + (bhq * S + qw + c) * 4);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      qop[m] = make_v8i(*reinterpret_cast<const uint4*>(qrow + 64 * m + 16 * hf),
                        *reinterpret_cast<const uint4*>(qrow + 64 * m + 32 + 16 * hf));
      qsc[m] = (int)((sw >> (8 * (2 * m + hf))) & 0xffu);
    }
  }
  // Wait for Q here (vmcnt 0, other counters untouched). Otherwise the loop's first use of Q carries
  // a conservative vector-memory wait that also waits for the tile prefetch issued just before it,
  // exposing the global-memory latency on every tile.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  RowState st;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.o[dt][i] = 0.f;
  st.nT = 0.f;
  st.nTL = -CB_LOG2_448;
  st.lsum = 0.f;

  // Tile it of the workgroup's key range is full for this wave when 64(it+1) <= e_w, half (first
  // 32-key block only) when 64it < e_w < 64(it+1), and outside the wave's range when 64it >= e_w.
  uint32_t psc = 0;
  if (ntiles > 0) {
    TILE_LOAD(sm[0], psc, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    store_scales<kLeaky>(sm[0], psc, tid);
  }
  __syncthreads();
  // One 64-key tile per iteration, double-buffered. The score MFMAs of tile it come first; then the
  // loads of tile it + 1 into the other buffer (last read before the barrier that ended iteration
  // it - 1); then the softmax and P.V. The first LDS read after those loads is the P.V operand read at
  // the end of the softmax, so the wait for them (which the compiler places before any later LDS
  // read) hides under the softmax.
  // Iteration it with its buffer known at compile time (s = it % 2), so that the LDS addresses of the
  // iteration are immediate offsets from per-lane bases; the loop is unrolled by two.
  auto step = [&](auto kslot, int it) {
    constexpr int s = decltype(kslot)::value;
    const int kt0 = it * CB_BN;
    const TileSmem& cur = sm[s];
    // The keys of this tile the wave attends: all 64 (full) or the first 32-key block (half); in the
    // ordinary causal variant also a completed block followed by the own block, masked per element
    // (own2), or the own block alone (own1).
    const bool full = kt0 + CB_BN <= e_w;
    const bool half = !kLeaky && !full && kt0 < e_w;
    const bool own2 = kLeaky && !full && kt0 < e_w;
    const bool own1 = kLeaky && wave_valid && kt0 == e_w;
    v16f sacc[2];
    if (full || own2)
      scores<true, kLeaky>(sacc, cur, qop, qsc, c, hf);
    else if (half || own1)
      scores<false, kLeaky>(sacc, cur, qop, qsc, c, hf);
    if (it + 1 < ntiles) TILE_LOAD(sm[s ^ 1], psc, kt0 + CB_BN);
    if (full)
      softmax_pv<true>(st, sacc, cur, scale_log2, c, hf, it == 0);
    else if (half)
      softmax_pv<false>(st, sacc, cur, scale_log2, c, hf, it == 0);
    else if (own2)
      softmax_pv<true, 1>(st, sacc, cur, scale_log2, c, hf, it == 0);
    else if (own1)
      softmax_pv<false, 0>(st, sacc, cur, scale_log2, c, hf, it == 0);
    // The next tile's loads (LDS and scale word) are complete here on every path; then its scales
    // are stored and the barrier publishes the tile.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (it + 1 < ntiles) store_scales<kLeaky>(sm[s ^ 1], psc, tid);
    __syncthreads();
  };
  for (int it = 0; it < ntiles; it += 2) {
    step(std::integral_constant<int, 0>{}, it);
    if (it + 1 < ntiles) step(std::integral_constant<int, 1>{}, it + 1);
  }

  // This lane's query row (used below only by valid waves, for which e_w = qw), derived here from
  // values the loop keeps live anyway, so that no row offset from before the loop has to be kept.
  int qr = e_w + c;
  asm("" : "+v"(qr));
  float la = st.lsum, lb = st.lsum;
  swap32f(la, lb);
  const float lc_tot = la + lb;       // l of the completed partial (both lane halves)
  const bool empty = (e_w == 0);      // rows 0..31 have no completed key

  if (kLeaky) {
    // O = acc / l and lse of the ordinary causal row (every row has at least its own key)
    if (!wave_valid) return;
    const float inv = 1.0f / lc_tot;
    const int64_t off = b * P.osb + (int64_t)qr * P.oss + hq * P.osh + 4 * hf;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = st.o[dt][4 * g + e] * inv;
        const int64_t o = off + 32 * dt + 8 * g;
        if (P.out_bf16) {
          uint2 pk;
          pk.x = f32_to_bf16(r[0]) | (f32_to_bf16(r[1]) << 16);
          pk.y = f32_to_bf16(r[2]) | (f32_to_bf16(r[3]) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(P.out) + o) = pk;
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(P.out) + o) = make_float4(r[0], r[1], r[2], r[3]);
        }
      }
    if (hf == 0 && P.lse_out) P.lse_out[bhq * S + qr] = (log2f(lc_tot) - st.nT) * 0.69314718055994530942f;
    return;
  } else if (!kFused) {
    if (!wave_valid) return;
    float* orow = P.o_c + (bhq * S + qr) * 128;
    const float inv = empty ? 0.f : 1.0f / lc_tot;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // Lane (c, hf), element 4g + r of tile dt: column d = 32dt + 8g + 4hf + r.
        const float4 val = make_float4(st.o[dt][4 * g] * inv, st.o[dt][4 * g + 1] * inv,
                                       st.o[dt][4 * g + 2] * inv, st.o[dt][4 * g + 3] * inv);
        *reinterpret_cast<float4*>(orow + 32 * dt + 8 * g + 4 * hf) = val;
      }
    if (hf == 0) P.lse_c[bhq * S + qr] = empty ? -INFINITY : (log2f(lc_tot) - st.nT) * 0.69314718055994530942f;
    return;
  } else {
    // ---- own block: keys qw .. qw+31, query qw + c sees keys up to itself ----------------------
    uint16_t* vown = reinterpret_cast<uint16_t*>(lds) + wave * (32 * 128);  // this wave's 32 x 128 bf16
    v16f so;
#pragma unroll
    for (int i = 0; i < 16; ++i) so[i] = 0.f;
    if (wave_valid) {
      // scores S^T = K_own Q^T on the same block-scaled FP8 MFMA as the completed blocks
      const uint8_t* krow = kc + (bhk * S + qw + c) * 128;
      const uint32_t ksw = *reinterpret_cast<const uint32_t*>(ks + (bhk * S + qw + c) * 4);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const v8i kop = make_v8i(*reinterpret_cast<const uint4*>(krow + 64 * m + 16 * hf),
                                 *reinterpret_cast<const uint4*>(krow + 64 * m + 32 + 16 * hf));
        const int ksc = (int)((ksw >> (8 * (2 * m + hf))) & 0xffu);
        so = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop, qop[m], so, 0, 0, 0, ksc, 0, qsc[m]);
      }
      // decode the token-normalised V rows of the block: lane -> key lane/2, 64 columns
      const int j = lane >> 1, d0 = (lane & 1) * 64;
      const uint8_t* vrow = P.vt + (bhk * S + qw + j) * 128 + d0;
      const float amp = e8m0_to_f32(P.vta[bhk * S + qw + j]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 w = *reinterpret_cast<const uint4*>(vrow + 16 * q);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
        uint32_t packed[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // v_cvt_pk_f32_fp8 decodes two OCP E4M3 codes exactly (every code checked on gfx950). An
          // E4M3 value times the amplitude has at most 4 significant bits, so the top 16 bits of
          // the fp32 product are its exact bf16.
          const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)ww[r], false);
          const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)ww[r], true);
          packed[2 * r] = (f2u(lo[0] * amp) >> 16) | (f2u(lo[1] * amp) & 0xffff0000u);
          packed[2 * r + 1] = (f2u(hi[0] * amp) >> 16) | (f2u(hi[1] * amp) & 0xffff0000u);
        }
        uint4* dst = reinterpret_cast<uint4*>(vown + j * 128 + d0 + 16 * q);
        dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
      }
    }
    __syncthreads();  // decoded rows visible to the whole wave
    if (!wave_valid) return;
    // softmax over the own block in the log2 domain; element i holds key 8(i/4) + 4hf + (i%4)
    float t[16];
    float mo = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = 8 * (i >> 2) + 4 * hf + (i & 3);
      t[i] = (j <= c) ? so[i] * scale_log2 : -INFINITY;
      mo = fmaxf(mo, t[i]);
    }
    float mo2 = mo;
    swap32f(mo, mo2);
    mo = fmaxf(mo, mo2);  // row max (key c itself is always visible)
    float pa[16];
    float lo = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      pa[i] = __builtin_amdgcn_exp2f(t[i] - mo);  // masked keys: exp2(-inf) = 0
      lo += pa[i];
    }
    float lo2 = lo;
    swap32f(lo, lo2);
    lo += lo2;
    // ---- merge weights through the log-sum-exps (log2 units) ----------------------------------
    const float l2c = empty ? -INFINITY : log2f(lc_tot) - st.nT;
    const float l2o = mo + log2f(lo);
    const float M = fmaxf(l2c, l2o);
    const float wc = empty ? 0.f : __builtin_amdgcn_exp2f(l2c - M);
    const float wo = __builtin_amdgcn_exp2f(l2o - M);
    const float inv = 1.0f / (wc + wo);
    const float fc = empty ? 0.f : wc * inv / lc_tot, fo = wo * inv / lo;
    const int q = qr;
    const int64_t off = b * P.osb + (int64_t)q * P.oss + hq * P.osh + 4 * hf;
    // ---- own O^T = V^T P^T in fp32 with v_mfma_f32_32x32x2_f32 ---------------------------------
    // Step u contracts the two keys 8(u/4) + (u%4) (k = 0) and 8(u/4) + 4 + (u%4) (k = 1): lane
    // (c, hf) supplies p of its query c for key k = hf, exactly pa[u]; as the A operand the same
    // lane supplies V^t[key k = hf][column 32dt + c]. The result has the layout of st.o[dt].
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      v16f oo;
#pragma unroll
      for (int e = 0; e < 16; ++e) oo[e] = 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int j = 8 * (u >> 2) + 4 * hf + (u & 3);
        const float a = u2f((uint32_t)vown[j * 128 + 32 * dt + c] << 16);
        oo = __builtin_amdgcn_mfma_f32_32x32x2f32(a, pa[u], oo, 0, 0, 0);
      }
      float rr[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) rr[e] = st.o[dt][e] * fc + oo[e] * fo;
      if (P.out_mxfp8) {
        // Block-scaled O (MXFP8, as the block-scaled O epilogue of cudnn-frontend PR #1088): one E8M0
        // per 32 columns 32dt .. 32dt+31 -- this lane holds 16 of them, lane ^ 32 the rest -- by the
        // same rule as the input quantiser (smallest k with amax <= 448 * 2^k), then the E4M3 codes of
        // x * 2^-k (exact scaling, round to nearest even).
        float am = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) am = vmax(am, fabsf(rr[e]));
        float am2 = am;
        swap32f(am, am2);
        am = vmax(am, am2);
        const int k = e8m0_exponent(am);
        const float m = pow2_neg(k);
        uint8_t* ob = reinterpret_cast<uint8_t*>(P.out);
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<uint32_t*>(ob + off + 32 * dt + 8 * g) =
              pack4_e4m3(rr[4 * g] * m, rr[4 * g + 1] * m, rr[4 * g + 2] * m, rr[4 * g + 3] * m);
        if (hf == 0) P.sf_o[(bhq * S + q) * 4 + dt] = (uint8_t)(k + 127);
        continue;
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = rr[4 * g + e];
        const int64_t o = off + 32 * dt + 8 * g;
        if (P.out_bf16) {
          uint2 pk;
          pk.x = f32_to_bf16(r[0]) | (f32_to_bf16(r[1]) << 16);
          pk.y = f32_to_bf16(r[2]) | (f32_to_bf16(r[3]) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(P.out) + o) = pk;
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(P.out) + o) = make_float4(r[0], r[1], r[2], r[3]);
        }
      }
    }
    if (hf == 0 && P.lse_out) P.lse_out[bhq * S + q] = (M + log2f(wc + wo)) * 0.69314718055994530942f;
  }
}

static AttnParams base_params(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                              const uint8_t* vc, const uint8_t* vcs, int B, int S, int Hq, int Hkv,
                              float softmax_scale) {
  AttnParams p{};
  p.qc = qc; p.qs = qs; p.kc = kc; p.ks = ks; p.vc = vc; p.vcs = vcs;
  p.S = S; p.Hq = Hq; p.Hkv = Hkv;
  p.n_qtiles = (S + CB_BM - 1) / CB_BM;
  p.n_pairs = B * Hq;
  p.xcd_pairs = (p.n_pairs % 8 == 0) ? p.n_pairs / 8 : 0;
  p.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
  return p;
}

hipError_t launch_attn_completed(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                                 const uint8_t* vc, const uint8_t* vcs, int B, int S, int Hq, int Hkv,
                                 float softmax_scale, float* o_c, float* lse_c, hipStream_t stream) {
  AttnParams p = base_params(qc, qs, kc, ks, vc, vcs, B, S, Hq, Hkv, softmax_scale);
  p.o_c = o_c;
  p.lse_c = lse_c;
  attn_kernel<MODE_COMPLETED><<<dim3((unsigned)(p.n_qtiles * p.n_pairs)), dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_attn_fused(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                             const uint8_t* vc, const uint8_t* vcs, const uint8_t* vt, const uint8_t* vta, int B,
                             int S, int Hq, int Hkv, float softmax_scale, void* out, int64_t osb, int64_t oss,
                             int64_t osh, int out_bf16, float* lse_out, hipStream_t stream, uint8_t* sf_o,
                             const uint16_t* qbf, int64_t qsb, int64_t qss, int64_t qsh) {
  AttnParams p = base_params(qc, qs, kc, ks, vc, vcs, B, S, Hq, Hkv, softmax_scale);
  p.qbf = qbf;
  p.qsb = qsb;
  p.qss = qss;
  p.qsh = qsh;
  p.vt = vt;
  p.vta = vta;
  p.out = out;
  p.osb = osb;
  p.oss = oss;
  p.osh = osh;
  p.out_bf16 = out_bf16;
  p.out_mxfp8 = sf_o != nullptr;
  p.sf_o = sf_o;
  p.lse_out = lse_out;
  attn_kernel<MODE_FUSED><<<dim3((unsigned)(p.n_qtiles * p.n_pairs)), dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_attn_leaky(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                             const uint8_t* vc, const uint8_t* vcs, int B, int S, int Hq, int Hkv, float softmax_scale,
                             void* out, int64_t osb, int64_t oss, int64_t osh, int out_bf16, float* lse_out,
                             hipStream_t stream) {
  AttnParams p = base_params(qc, qs, kc, ks, vc, vcs, B, S, Hq, Hkv, softmax_scale);
  p.out = out;
  p.osb = osb;
  p.oss = oss;
  p.osh = osh;
  p.out_bf16 = out_bf16;
  p.lse_out = lse_out;
  attn_kernel<MODE_LEAKY><<<dim3((unsigned)(p.n_qtiles * p.n_pairs)), dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace mxfa
