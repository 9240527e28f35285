// attn_own_block.hip -- the own-block partial of leak-free causal MXFP8 attention, gfx950.
//
// TransformerEngine PR #3865, "Description", second bullet: each query's own 32-token block (at most
// 32 keys) is computed on a token-normalised copy of V (one power-of-two amplitude per token) and
// merged with the completed-block partial through the log-sum-exps. Reading used here: scores from
// the decoded rowwise MXFP8 Q/K (the operands the completed blocks use), softmax and P.V in fp32 with
// P not quantised, V decoded from the token-normalised codes.
//
// One wave per 32-query block (the block's own 32 keys), four blocks per workgroup; per wave:
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys on the rows, queries on the columns), the Q and K
//    codes decoded to bf16 in registers. An E4M3 value times a power of two has at most 4 significant
//    bits, so the decoded value is a bf16 value (for scale bytes >= 3; below that it can fall under
//    bf16's finest step, 2^-133) and the products are exact; the MFMA sums them in fp32.
//  * Masked softmax of each query's column in fp32, in the log2 domain.
//  * O = (P / l) V on v_mfma_f32_32x32x16_bf16 without rounding P: each p / l is split exactly into
//    three bf16 parts (8 significant bits each) that go through the same product; V decoded to bf16
//    in LDS, transposed (exact under the same condition on its amplitude byte). O and the lse written
//    once, O in whole 128-byte row pieces.
// HBM-bound: per query row it reads 132 code and scale bytes and writes 516 bytes, plus the block's
// K and V rows, shared by its 32 queries.
#include "device_common.h"
#include "launch.h"

namespace mxfa {

typedef __bf16 v8bf_o __attribute__((ext_vector_type(8)));
constexpr int OB_VT_PITCH = 36;  // bf16 per V^T row in LDS: 32 keys + 4 (spreads the rows over the banks)

// Eight E4M3 codes (byte e -> element e) times the power of two sc, as bf16 (exact, see above).
__device__ __forceinline__ v8bf_o decode8_bf16(uint2 codes, float sc) {
  uint32_t w[4];
  const uint32_t cw[2] = {codes.x, codes.y};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[h], false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[h], true);
    w[2 * h] = (f2u(lo[0] * sc) >> 16) | (f2u(lo[1] * sc) & 0xffff0000u);
    w[2 * h + 1] = (f2u(hi[0] * sc) >> 16) | (f2u(hi[1] * sc) & 0xffff0000u);
  }
  return __builtin_bit_cast(v8bf_o, make_uint4(w[0], w[1], w[2], w[3]));
}

// x combined with the value of lane ^ 32: v_permlane32_swap of two copies of x leaves every lane its
// own value in one output and its partner's in the other.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  return fmaxf(u2f(r[0]), u2f(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  return u2f(r[0]) + u2f(r[1]);
}

__global__ __launch_bounds__(256) void own_block_kernel(const uint8_t* __restrict__ qc, const uint8_t* __restrict__ qs,
                                                        const uint8_t* __restrict__ kc, const uint8_t* __restrict__ ks,
                                                        const uint8_t* __restrict__ vt,
                                                        const uint8_t* __restrict__ vta, int S, int Hq, int Hkv,
                                                        float scale, float* __restrict__ o,
                                                        float* __restrict__ lse) {
  __shared__ __align__(16) uint16_t vcols[4][128 * OB_VT_PITCH];  // each wave's decoded V^T, bf16
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 31, hf = lane >> 5;
  const int hq = blockIdx.y, b = blockIdx.z, hk = hq / (Hq / Hkv);
  const int j0 = 32 * (4 * (int)blockIdx.x + wave);  // first query (and key) of this wave's block
  const bool valid = j0 < S;                          // S % 32 == 0: whole blocks only
  const int64_t qrow0 = ((int64_t)b * Hq + hq) * S + j0;
  const int64_t krow0 = ((int64_t)b * Hkv + hk) * S + j0;
  uint16_t* vown = vcols[wave];
  v16f so;
#pragma unroll
  for (int i = 0; i < 16; ++i) so[i] = 0.f;
  if (valid) {
    // Lane (c, hf) supplies, for step s, columns 16s + 8hf + [0, 8) of key row c (A) and of query row c
    // (B); their scale is byte s / 2 of the row's four.
    const uint8_t* qr = qc + (qrow0 + c) * 128 + 8 * hf;
    const uint8_t* kr = kc + (krow0 + c) * 128 + 8 * hf;
    const uint32_t qsw = *reinterpret_cast<const uint32_t*>(qs + (qrow0 + c) * 4);
    const uint32_t ksw = *reinterpret_cast<const uint32_t*>(ks + (krow0 + c) * 4);
    uint2 qcod[8], kcod[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qcod[s] = *reinterpret_cast<const uint2*>(qr + 16 * s);
      kcod[s] = *reinterpret_cast<const uint2*>(kr + 16 * s);
    }
    // Decode the token-normalised V of the block into V^T (row d holds the 32 keys' values of column
    // d): item w = (keys 4a .. 4a+3, a = w % 8; columns 8bb .. 8bb+7, bb = w / 8), two items per lane.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int w = lane + 64 * h, a = w & 7, bb = w >> 3;
      const uint32_t amps = *reinterpret_cast<const uint32_t*>(vta + krow0 + 4 * a);
      uint32_t pk[2][8];  // column 8bb + t: bf16 of keys 4a + 2x (low half) and 4a + 2x + 1 (high half)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint2 cw = *reinterpret_cast<const uint2*>(vt + (krow0 + 4 * a + r) * 128 + 8 * bb);
        const float amp = e8m0_to_f32((amps >> (8 * r)) & 0xffu);
        const uint32_t cc[2] = {cw.x, cw.y};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)cc[hh], false);
          const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)cc[hh], true);
          const float f[4] = {lo[0] * amp, lo[1] * amp, hi[0] * amp, hi[1] * amp};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t& d = pk[r >> 1][4 * hh + q];
            d = (r & 1) ? (d | (f2u(f[q]) & 0xffff0000u)) : (f2u(f[q]) >> 16);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < 8; ++t)
        *reinterpret_cast<uint2*>(vown + (8 * bb + t) * OB_VT_PITCH + 4 * a) = make_uint2(pk[0][t], pk[1][t]);
      // one item at a time: the second item's loads are issued after the first item's writes
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int sb = 8 * (s >> 1);
      const v8bf_o ka = decode8_bf16(kcod[s], e8m0_to_f32((ksw >> sb) & 0xffu));
      const v8bf_o qb = decode8_bf16(qcod[s], e8m0_to_f32((qsw >> sb) & 0xffu));
      so = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb, so, 0, 0, 0);
    }
  }
  __syncthreads();  // the decoded V^T is visible to the whole wave
  if (!valid) return;
  // Lane (c, hf), element i: key 8(i/4) + 4hf + i%4 of query c; softmax over keys <= c (log2 domain).
  const float scale_log2 = scale * 1.4426950408889634f;
  float t[16];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int j = 8 * (i >> 2) + 4 * hf + (i & 3);
    t[i] = (j <= c) ? so[i] * scale_log2 : -INFINITY;
    m = fmaxf(m, t[i]);
  }
  m = halves_max(m);  // key c itself is visible, so m is finite
  float pa[16];
  float l = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    pa[i] = __builtin_amdgcn_exp2f(t[i] - m);  // masked keys: exp2(-inf) = 0
    l += pa[i];
  }
  l = halves_sum(l);
  const float inv = 1.0f / l;
  // p / l split exactly into three bf16 parts (each the next 8 significant bits; truncation leaves an
  // exact remainder), as pairs of elements (2k, 2k + 1).
  uint32_t ph[8], pm[8], pl[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint32_t hb[2], mb[2], lb[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float x = pa[2 * k + e] * inv;
      hb[e] = f2u(x) & 0xffff0000u;
      const float r = x - u2f(hb[e]);
      mb[e] = f2u(r) & 0xffff0000u;
      lb[e] = f2u(r - u2f(mb[e])) & 0xffff0000u;
    }
    ph[k] = (hb[0] >> 16) | hb[1];
    pm[k] = (mb[0] >> 16) | mb[1];
    pl[k] = (lb[0] >> 16) | lb[1];
  }
  // O = (P / l) V on v_mfma_f32_32x32x16_bf16, one 32-column tile dt at a time, two 16-key steps of
  // three products each. Step kk's contraction slot 8g + e is key 16kk + 8(e/4) + 4g + e%4: lane
  // (c, hf) supplies p of query c for its elements 8kk + e (A) and V^T row 32dt + c at keys
  // 16kk + 4hf + [0, 4) and 16kk + 8 + 4hf + [0, 4) (B). Element i of the result is query
  // 8(i/4) + 4hf + i%4, column 32dt + c, so each store writes two whole 128-byte row pieces.
  auto pair4 = [](const uint32_t* w) { return __builtin_bit_cast(v8bf_o, make_uint4(w[0], w[1], w[2], w[3])); };
  const v8bf_o ah[2] = {pair4(ph), pair4(ph + 4)}, am[2] = {pair4(pm), pair4(pm + 4)},
               al[2] = {pair4(pl), pair4(pl + 4)};
  float* ocol = o + qrow0 * 128 + c;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    v16f oo;
#pragma unroll
    for (int e = 0; e < 16; ++e) oo[e] = 0.f;
    const uint16_t* vrow = vown + (32 * dt + c) * OB_VT_PITCH + 4 * hf;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint2 v0 = *reinterpret_cast<const uint2*>(vrow + 16 * kk);
      const uint2 v1 = *reinterpret_cast<const uint2*>(vrow + 16 * kk + 8);
      const v8bf_o vb = __builtin_bit_cast(v8bf_o, make_uint4(v0.x, v0.y, v1.x, v1.y));
      oo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[kk], vb, oo, 0, 0, 0);
      oo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am[kk], vb, oo, 0, 0, 0);
      oo = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[kk], vb, oo, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) ocol[(8 * (i >> 2) + 4 * hf + (i & 3)) * 128 + 32 * dt] = oo[i];
    __builtin_amdgcn_sched_barrier(0);  // one tile's accumulator at a time (register pressure)
  }
  if (hf == 0) lse[qrow0 + c] = (m + log2f(l)) * 0.69314718055994530942f;
}

hipError_t launch_attn_own_block(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks,
                                 const uint8_t* vt, const uint8_t* vta, int B, int S, int Hq, int Hkv,
                                 float softmax_scale, float* o_o, float* lse_o, hipStream_t stream) {
  dim3 grid((unsigned)((S / 32 + 3) / 4), (unsigned)Hq, (unsigned)B);
  own_block_kernel<<<grid, dim3(256), 0, stream>>>(qc, qs, kc, ks, vt, vta, S, Hq, Hkv, softmax_scale, o_o, lse_o);
  return hipGetLastError();
}

}  // namespace mxfa
