// fs_device.h -- device-side building blocks of the FlashSampling kernels (gfx950).
//
// Noise: Philox4x32-10 keyed on (seed, step, row, vocab id) and the transform of
// a 32-bit word r into standard Gumbel noise through u = (r+1)/(2^32+1),
// g = -log(-log u).  [readus.org FlashSampling summary, code guide sections 2
// (Philox keyed by master seed and coordinates) and 3 (the u formula, which keeps
// u strictly inside (0, 1))]
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fsk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64-bit multiplies and xors; the key advances by a Weyl step after each
// round.  One call yields the four words of four consecutive vocab ids.
// The products are formed as separate high and low 32-bit multiplies: the
// fused 64-bit form (v_mad_u64_u32 with a scalar operand, which writes a carry
// to scalar registers) stalled the W stream measurably on gfx950, the split
// form does not.
// ---------------------------------------------------------------------------
struct Philox4 {
  uint32_t w[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t k0, uint32_t k1, uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    // one 32 x 32 -> 64-bit multiply each (a single v_mad_u64_u32) rather than
    // separate high and low products
    const uint64_t pa = (uint64_t)0xD2511F53u * c0, pb = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t hi_a = (uint32_t)(pa >> 32), lo_a = (uint32_t)pa;
    const uint32_t hi_b = (uint32_t)(pb >> 32), lo_b = (uint32_t)pb;
    const uint32_t n0 = hi_b ^ c1 ^ k0;
    const uint32_t n2 = hi_a ^ c3 ^ k1;
    c1 = lo_b;
    c3 = lo_a;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  Philox4 out;
  out.w[0] = c0;
  out.w[1] = c1;
  out.w[2] = c2;
  out.w[3] = c3;
  return out;
}

// Counter of vocab quad (gv >> 2) of row b at a step: (gv >> 2, b, step lo, step hi).
struct NoiseKey {
  uint32_t seed_lo, seed_hi, step_lo, step_hi;
};

__device__ __forceinline__ Philox4 noise_quad(const NoiseKey& k, uint32_t quad, uint32_t row) {
  return philox4x32_10(k.seed_lo, k.seed_hi, quad, row, k.step_lo, k.step_hi);
}

// ---------------------------------------------------------------------------
// Gumbel noise of one word.  With m = r + 1 (r < 2^31) or m = 2^32 - r
// (r >= 2^31), t = m * 2^-32 lies in (0, 1/2] and is the smaller of u and 1-u
// (the factor 2^32/(2^32+1) is below fp32 resolution).  E = -ln u is then
// -ln t (lower half) or -ln(1 - t) (upper half); the latter uses its Taylor
// series for t < 1/16 (remainder below t * 2^-35) so that E keeps full
// relative precision as u -> 1, where the largest noise values come from.
// Every word gives a finite value in [-3.0992, 22.181].
// ---------------------------------------------------------------------------
__device__ __forceinline__ float fast_ln(float x) {  // hardware log2, x normal and > 0
  return __builtin_amdgcn_logf(x) * 0.693147180559945309f;
}

__device__ __forceinline__ float gumbel_from_bits(uint32_t r) {
  const bool upper = r >= 0x80000000u;
  const uint32_t m = upper ? (0u - r) : (r + 1u);
  const float t = (float)m * 0x1p-32f;
  // -ln(1 - t) / t = sum_{n>=1} t^(n-1) / n, eight terms
  float poly = 0.125f;
  poly = __builtin_fmaf(poly, t, 0.142857142857142857f);
  poly = __builtin_fmaf(poly, t, 0.166666666666666667f);
  poly = __builtin_fmaf(poly, t, 0.2f);
  poly = __builtin_fmaf(poly, t, 0.25f);
  poly = __builtin_fmaf(poly, t, 0.333333333333333333f);
  poly = __builtin_fmaf(poly, t, 0.5f);
  poly = __builtin_fmaf(poly, t, 1.0f);
  const float larg = upper ? (1.0f - t) : t;
  const float ln_arg = fast_ln(larg);
  const float e = (upper && t < 0.0625f) ? t * poly : -ln_arg;
  return -fast_ln(e);
}

// x from lane (lane ^ OFF) of the wave, OFF a power of two up to 32, on the
// vector ALU: DPP moves within a row of 16 lanes (quad permutes for 1 and 2,
// row shifts either way for 4, a rotation by half a row for 8) and gfx950's
// permlane swaps across rows (for 16 and 32: one swap of x with itself leaves
// lane l's partner in one of the two results).  __shfl_xor goes through the
// LDS crossbar, a round trip per exchange, and the reductions and list merges
// at the end of a tile are chains of exchanges.  Every lane of the wave must
// be active.
template <int OFF>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x) {
  const int lane = threadIdx.x & 63;
  if constexpr (OFF == 1) {
    return __builtin_amdgcn_update_dpp(0u, x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  } else if constexpr (OFF == 2) {
    return __builtin_amdgcn_update_dpp(0u, x, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  } else if constexpr (OFF == 4) {
    const uint32_t up = __builtin_amdgcn_update_dpp(0u, x, 0x104, 0xF, 0xF, false);  // row_shl:4 (from lane + 4)
    const uint32_t dn = __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false);  // row_shr:4 (from lane - 4)
    return (lane & 4) ? dn : up;
  } else if constexpr (OFF == 8) {
    return __builtin_amdgcn_update_dpp(0u, x, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & 16) ? r[0] : r[1];
  } else {
    static_assert(OFF == 32, "lane distances 1, 2, 4, 8, 16 and 32");
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane & 32) ? r[0] : r[1];
  }
}

template <int OFF>
__device__ __forceinline__ uint64_t lane_xor64(uint64_t x) {
  return (uint64_t)lane_xor<OFF>((uint32_t)x) | ((uint64_t)lane_xor<OFF>((uint32_t)(x >> 32)) << 32);
}

template <int OFF>
__device__ __forceinline__ float lane_xor_f(float x) {
  return __uint_as_float(lane_xor<OFF>(__float_as_uint(x)));
}

// ---------------------------------------------------------------------------
// (value, index) maximizer with the lowest-index tie rule.  NaN values never
// win: they fail every comparison.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool beats(float va, int32_t ia, float vb, int32_t ib) {
  return va > vb || (va == vb && ia < ib);
}

__device__ __forceinline__ void merge_best(float& v, int32_t& i, float ov, int32_t oi) {
  if (beats(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

template <int OFF>
__device__ __forceinline__ void merge_best_xor(float& v, int32_t& i) {
  merge_best(v, i, lane_xor_f<OFF>(v), (int32_t)lane_xor<OFF>((uint32_t)i));
}

// Wave-wide maximizer: afterwards every lane holds the wave's best (value,
// index).  Every lane of the wave must be active.
__device__ __forceinline__ void wave_best(float& v, int32_t& i) {
  merge_best_xor<32>(v, i);
  merge_best_xor<16>(v, i);
  merge_best_xor<8>(v, i);
  merge_best_xor<4>(v, i);
  merge_best_xor<2>(v, i);
  merge_best_xor<1>(v, i);
}

// Online log-sum-exp state (running max m, sum of exp(x - m)).
__device__ __forceinline__ void lse_push(float& m, float& s, float x) {
  if (x == -INFINITY) return;
  if (x > m) {
    s = s * __expf(m - x) + 1.0f;
    m = x;
  } else {
    s += __expf(x - m);
  }
}

__device__ __forceinline__ void lse_merge(float& m, float& s, float om, float os) {
  const float mm = fmaxf(m, om);
  if (mm == -INFINITY) {
    m = -INFINITY;
    s = 0.0f;
    return;
  }
  s = (m == -INFINITY ? 0.0f : s * __expf(m - mm)) + (om == -INFINITY ? 0.0f : os * __expf(om - mm));
  m = mm;
}

// ---------------------------------------------------------------------------
// Top-k keys: one 64-bit word per (score, id) whose unsigned order is the
// selection order -- higher score first, lower id first among equal scores.
// High word: the score's bits mapped to an unsigned order (sign flipped for
// positives, all bits inverted for negatives; -0 folded onto +0); low word:
// the id's complement.  0 marks an empty slot: every real key exceeds it.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_bits(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_bits_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ uint64_t topk_key(float s, int32_t id) {
  return ((uint64_t)order_bits(s) << 32) | (uint64_t)(~(uint32_t)id);
}

__device__ __forceinline__ float topk_key_score(uint64_t key) { return order_bits_inv((uint32_t)(key >> 32)); }
__device__ __forceinline__ int32_t topk_key_id(uint64_t key) { return (int32_t)(~(uint32_t)key); }

__device__ __forceinline__ bool mask_allows(const uint32_t* __restrict__ mask_row, int64_t gv) {
  return (mask_row[gv >> 5] >> (uint32_t)(gv & 31)) & 1u;
}

}  // namespace fsk
