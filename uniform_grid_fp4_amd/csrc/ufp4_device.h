// Device helpers for the UFP4 kernels (gfx950): Philox4x32-10, bf16 unpack,
// the 16-point Walsh-Hadamard butterfly, and rounding onto the two 4-bit
// grids with the nibble encoding.
//
// Method: "Rethinking Shrinkage Bias in LLM FP4 Pretraining" (arXiv
// 2606.20381), paperlayer.ai summary, section 2 ("FP4 formats", "Blockwise
// quantization", "Rounding rules", "Random Hadamard transforms").
//
// Every function here is exact FP32 arithmetic in a fixed order; the library
// is built with -ffp-contract=off so no multiply and add are fused.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ufp4 {

enum { kGridUniform = 0, kGridE2M1 = 1, kGridE2M1Max2 = 2 };

// Largest normalized magnitude g of a grid: the block absmax maps to g.
// Range-restricted E2M1 keeps the E2M1 levels up to 2.0 (and their bit
// patterns), so it shares E2M1's rounding below 2.
template <int GRID>
__host__ __device__ constexpr float grid_g() {
  return GRID == kGridUniform ? 7.0f : (GRID == kGridE2M1 ? 6.0f : 2.0f);
}
enum { kRoundRTNE = 0, kRoundSR = 1 };

// ---------------------------------------------------------------------------
// Philox4x32-10, Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3" (SC'11): ten rounds of two 32x32->64 products of counter
// words 0 and 2 with the published multipliers, the high halves xored with
// the other two words and the key; the key advances by the published Weyl
// increments after each round.  The key is wave-uniform, so its schedule stays
// in scalar registers.
// ---------------------------------------------------------------------------
struct U32x4 {
  uint32_t w[4];
};

__device__ __forceinline__ U32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    // three-input xors in one v_bitop3_b32 each (truth table 0x96)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  U32x4 o;
  o.w[0] = c0;
  o.w[1] = c1;
  o.w[2] = c2;
  o.w[3] = c3;
  return o;
}

// ---------------------------------------------------------------------------
// bf16 -> fp32 (exact), with the RHT sign folded into the sign bit.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w, uint32_t sgn) {
  return __uint_as_float((w << 16) ^ sgn);
}
__device__ __forceinline__ float bf16_hi(uint32_t w, uint32_t sgn) {
  return __uint_as_float((w & 0xFFFF0000u) ^ sgn);
}

// Sign bit (bit 31) applied to element j when bit j of the mask is set.
__device__ __forceinline__ uint32_t sign_bit(uint32_t mask, int j) {
  return ((mask >> j) & 1u) << 31;
}

// Unnormalised Sylvester-order Walsh-Hadamard butterfly of one block, in
// place: stages h = 1, 2, 4, 8; pair (i, i+h) with (i & h) == 0 becomes
// (v_i + v_{i+h}, v_i - v_{i+h}), each rounded to FP32.
__device__ __forceinline__ void fwht16(float (&v)[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const float a = v[i];
        const float b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Rounding a normalised value t (|t| <= g up to one ulp) to a magnitude index.
// ---------------------------------------------------------------------------
// E2M1 grid {0,.5,1,1.5,2,3,4,6}, RTNE with ties to the even index: within
// each binade the spacing is constant (0.5 below 2, 1 on [2,4), 2 on [4,6]),
// so the same magic-constant add at that binade's spacing rounds half to even,
// and index = (rounded value / spacing) + binade offset preserves parity.
__device__ __forceinline__ uint32_t e2m1_rtne(float m) {
  const bool lo = m < 2.0f;
  const bool mid = m < 4.0f;
  const float magic = lo ? 6291456.0f : (mid ? 12582912.0f : 25165824.0f);
  const uint32_t off = lo ? 0u : (mid ? 2u : 4u);
  return (__float_as_uint(m + magic) - __float_as_uint(magic)) + off;
}

// Stochastic rounding on E2M1: lo = largest level <= m, f = position of m
// between lo and the next level (exact), round up iff u < floor(f * 2^32).
__device__ __forceinline__ uint32_t e2m1_sr(float m, uint32_t u) {
  m = fminf(m, 6.0f);
  const bool lo = m < 2.0f;
  const bool mid = m < 4.0f;
  const float inv = lo ? 2.0f : (mid ? 1.0f : 0.5f);   // 1 / spacing, exact
  const uint32_t off = lo ? 0u : (mid ? 2u : 4u);
  const float q = m * inv;                             // exact
  const float fl = floorf(q);
  const float f = q - fl;
  const uint32_t F = (uint32_t)(f * 4294967296.0f);
  return (uint32_t)fl + off + (u < F ? 1u : 0u);
}

// ---------------------------------------------------------------------------
// Packing eight results into one word of nibbles (element 2i in the low
// nibble of byte i), SWAR style.
// ---------------------------------------------------------------------------
// Byte 0 of each of four registers -> one word [b0(a) b0(b) b0(c) b0(d)].
__device__ __forceinline__ uint32_t gather_b0(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_amdgcn_perm(b, a, 0x0C0C0400u) | __builtin_amdgcn_perm(d, c, 0x04000C0Cu);
}
// Byte 3 of each of four registers.
__device__ __forceinline__ uint32_t gather_b3(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_amdgcn_perm(b, a, 0x0C0C0703u) | __builtin_amdgcn_perm(d, c, 0x07030C0Cu);
}
// Even elements' low nibbles in the low halves of the bytes, odd elements' in
// the high halves: byte i = e[i] & 15 | (o[i] & 15) << 4.
__device__ __forceinline__ uint32_t interleave_nibbles(uint32_t even, uint32_t odd) {
  return (even & 0x0F0F0F0Fu) | ((odd << 4) & 0xF0F0F0F0u);
}
// Sign word: bit 7 of byte i of se/so (sign of element 2i / 2i+1) moved to
// bit 3 / bit 7 of byte i.
__device__ __forceinline__ uint32_t interleave_signs(uint32_t se, uint32_t so) {
  return (so & 0x80808080u) | ((se >> 4) & 0x08080808u);
}
// Sign-magnitude nibbles with the zero rule: the sign bit survives only where
// the magnitude is non-zero (m + 7 carries into bit 3 exactly when m >= 1,
// and never into the next nibble since m <= 7).
__device__ __forceinline__ uint32_t apply_signs(uint32_t mags, uint32_t signs) {
  return (signs & (mags + 0x77777777u)) | mags;
}
// Four-bit two's complement nibbles (values -7..7) -> sign-magnitude.  A
// negative nibble v has magnitude (~v & 15) + 1 <= 7 (no carry out); a zero
// stays zero, so no negative zero can appear.
__device__ __forceinline__ uint32_t twos_to_signmag(uint32_t w) {
  const uint32_t sg = w & 0x88888888u;
  const uint32_t one = sg >> 3;
  const uint32_t mag = (w ^ (one * 15u)) + one;
  return mag | sg;
}

// ---------------------------------------------------------------------------
// One block of 16 values already in registers (after bf16 unpack and the sign
// flip).  If RHT, v holds d_j * x_j and the butterfly runs here; the 1/4 of
// the orthonormal transform is folded into the reciprocal (exact: both are
// powers of two and every butterfly output of bf16 inputs is a multiple of
// 2^-133, so z/4 is exact).  Produces two 32-bit words of 8 nibbles (element
// 0 in the low nibble of word 0) and the FP32 block scale.
// idx0 is the SR index of element 0 of the block; its 16 elements use the
// four Philox outputs of counters idx0/4 .. idx0/4 + 3.
// ---------------------------------------------------------------------------
template <int GRID, int RND, bool RHT>
__device__ __forceinline__ void quantize_block(float (&v)[16], uint64_t idx0, uint32_t seed_lo,
                                               uint32_t seed_hi, uint32_t stream_id,
                                               uint32_t &w0, uint32_t &w1, float &scale) {
  if (RHT) fwht16(v);
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const float s = RHT ? amax * 0.25f : amax;   // exact
  scale = s;
  constexpr float g = grid_g<GRID>();
  float post;
  if (s >= 0x1p-64f) {
    const float r = g / s;                     // correctly rounded division
    post = RHT ? r * 0.25f : r;                // exact: r >= 7 * 2^-125
  } else {
    // 0 <= s < 2^-64: normalise with y * 2^64 and s * 2^64 (exact).  For
    // s == 0 all values are +-0 and every index is 0 whatever post is.
    const float r = (s > 0.0f) ? g / (s * 0x1p64f) : 0.0f;
    post = r;
    const float pre = RHT ? 0x1p62f : 0x1p64f; // (z / 4) * 2^64 = z * 2^62
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = v[j] * pre;
  }
  uint32_t rnd[16];
  if (RND == kRoundSR) {
    const uint64_t q0 = idx0 >> 2;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint64_t q = q0 + (uint64_t)c;
      const U32x4 o = philox4x32_10((uint32_t)q, (uint32_t)(q >> 32), stream_id, 0u,
                                    seed_lo, seed_hi);
#pragma unroll
      for (int j = 0; j < 4; ++j) rnd[4 * c + j] = o.w[j];
    }
  }
  float t[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) t[j] = v[j] * post;
  uint32_t words[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float *th = t + 8 * h;
    if (GRID == kGridUniform && RND == kRoundRTNE) {
      // Signed round half to even of t: adding 1.5 * 2^23 leaves round(t) in
      // the low mantissa bits, as a two's complement byte.
      uint32_t u[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) u[j] = __float_as_uint(th[j] + 12582912.0f);
      const uint32_t w = interleave_nibbles(gather_b0(u[0], u[2], u[4], u[6]),
                                            gather_b0(u[1], u[3], u[5], u[7]));
      words[h] = twos_to_signmag(w);
    } else {
      uint32_t k[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float m = fabsf(th[j]);
        const uint32_t r = rnd[8 * h + j];
        if (GRID == kGridUniform) {
          // k = floor(m) + (r < F); mc - floor(mc) is exact for 0 <= mc <= 7 and
          // is what v_fract_f32 returns there, and the truncating conversion
          // is floor(mc)
          const float mc = fminf(m, 7.0f);
          const uint32_t F = (uint32_t)(__builtin_amdgcn_fractf(mc) * 4294967296.0f);
          k[j] = (uint32_t)mc + (r < F ? 1u : 0u);
        } else {
          // m <= g up to one ulp; RTNE rounds that ulp back to g, SR must not
          // round past the top level
          k[j] = (RND == kRoundSR) ? e2m1_sr(GRID == kGridE2M1Max2 ? fminf(m, 2.0f) : m, r)
                                   : e2m1_rtne(m);
        }
      }
      const uint32_t mags = interleave_nibbles(gather_b0(k[0], k[2], k[4], k[6]),
                                               gather_b0(k[1], k[3], k[5], k[7]));
      const uint32_t signs = interleave_signs(
          gather_b3(__float_as_uint(th[0]), __float_as_uint(th[2]), __float_as_uint(th[4]),
                    __float_as_uint(th[6])),
          gather_b3(__float_as_uint(th[1]), __float_as_uint(th[3]), __float_as_uint(th[5]),
                    __float_as_uint(th[7])));
      words[h] = apply_signs(mags, signs);
    }
  }
  w0 = words[0];
  w1 = words[1];
}

}  // namespace ufp4
