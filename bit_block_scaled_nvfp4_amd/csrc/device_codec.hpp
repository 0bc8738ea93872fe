// device_codec.hpp -- gfx950 device primitives for NVFP4: E4M3 / E2M1 codecs,
// Philox4x32-10, the 16-point sign-randomised Hadamard butterflies and
// wavefront reductions.
//
// The element and scale formats are OCP MX E2M1 and OCP FP8 E4M3FN; the
// pages ("NVIDIA acelera o pre-treinamento de LLM: NVFP4 no Blackwell ...",
// section "Por Que Cada Porcento E Importante") only fix a 4-bit element with
// its own scaling scheme.  Encoders here work on IEEE-754 bit patterns so that
// each step costs a few integer VALU ops per element.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// ---------------------------------------------------------------------------
// BF16 pairs
// ---------------------------------------------------------------------------

// A dword holding two BF16 values (element 2j in the low half) widens exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// E4M3FN block scale (only non-negative codes 0x00..0x7E are produced)
// ---------------------------------------------------------------------------

// Value of a non-negative E4M3FN code.  Codes below 8 are subnormal
// (m * 2^-9); above, the 7 code bits shifted to the FP32 exponent/mantissa
// position plus an exponent rebias of 127 - 7 give the value directly.
__device__ __forceinline__ float e4m3_value(uint32_t s) {
  return (s < 8u) ? (float)s * 0x1p-9f : __uint_as_float((s + (120u << 3)) << 20);
}

// y >= 0 -> E4M3FN code, round to nearest even, saturating at 448 (0x7E).
// Normal range: add the rounding bias below the 3 kept mantissa bits (ties to
// even through the kept LSB); a carry out of the mantissa bumps the exponent,
// which is the correct rounding.  Subnormal range (< 2^-6): round y * 2^9 to
// an integer; 8 there is the code of 2^-6.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  y = fminf(y, 448.0f);
  if (y < 0x1p-6f) return (uint32_t)__builtin_rintf(y * 512.0f);
  uint32_t u = __float_as_uint(y);
  return ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - (120u << 3);
}

// ---------------------------------------------------------------------------
// E2M1 element encode
// ---------------------------------------------------------------------------

// Eight values -> eight RNE codes packed into a dword (element j in nibble j)
// with gfx950's FP32 -> FP4 converter at unit scale, two values per
// instruction.  Its results equal the oracle's round-to-nearest-even encoder
// on every non-NaN FP32 input: tests/test_hw_converters.py sweeps all 2^32
// bit patterns through this function on the GPU.
__device__ __forceinline__ uint32_t e2m1_rne8(const float *q) {
  // The four converts write bytes 0..3, so the word's initial value never
  // shows; any live register will do (no zeroing move needed).
  uint32_t w = __float_as_uint(q[0]);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[0], q[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[2], q[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[4], q[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[6], q[7], 1.0f, 3);
  return w;
}

// Stochastic rounding onto the same grid: with f the rounding fraction of
// |q| (clamped to 6) between its grid neighbours and F = floor(f * 2^22),
// the magnitude rounds up iff 64 u < F for the element's 16-bit word u.
// gfx950's stochastic-rounding converter adds the top 22 bits of a random
// operand to the 22 fraction bits it keeps below the E2M1 point and rounds
// up on the carry: with ~(u << 16) as that operand it rounds up iff
// F + 2^22 - 1 - 64 u >= 2^22, which is the rule above.  Its two lanes share
// one random operand (the high lane sees it shifted left by one), so each
// conversion carries one element, the other lane converting +0 (code 0):
// even elements in the low lane with ~(u << 16); odd elements in the high
// lane with ((~w) >> 1) | 0x7FFF, whose left shift by one has ~u in its top
// 16 bits and ones below (w the Philox word, u its high half).  Sign,
// saturation and signed zeros come out as the rule has them.
// tests/test_hw_converters.py checks every FP32 value at the words around
// its rounding threshold against the oracle (both lanes); the rule is
// monotone in u, so that covers every word.  Element j of the 8 uses 16-bit
// half (j & 1) of word j / 2 of r; element j lands in nibble j.
typedef float float2_v __attribute__((ext_vector_type(2)));
// Byte 0 of the result: the code of q_even in the low nibble and of q_odd in
// the high one (words u = w & 0xFFFF and w >> 16).  This build does not tie
// the converter's destination to its first operand, so only the byte it is
// told to write (byte 0 here) is defined; the caller gathers the bytes.
__device__ __forceinline__ uint32_t e2m1_sr_pair(float q_even, float q_odd, uint32_t w) {
  const uint32_t nw = ~w;
  const float2_v lo = {q_even, 0.0f}, hi = {0.0f, q_odd};
  return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, lo, (nw << 16) | 0xFFFFu, 1.0f, 0) |
         __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, hi, (nw >> 1) | 0x7FFFu, 1.0f, 0);
}
__device__ __forceinline__ uint32_t e2m1_sr8(const float *q, uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  const uint32_t x0 = e2m1_sr_pair(q[0], q[1], w0), x1 = e2m1_sr_pair(q[2], q[3], w1);
  const uint32_t x2 = e2m1_sr_pair(q[4], q[5], w2), x3 = e2m1_sr_pair(q[6], q[7], w3);
  const uint32_t a = __builtin_amdgcn_perm(x1, x0, 0x0C0C0400u);  // [x0.b0, x1.b0, 0, 0]
  const uint32_t b = __builtin_amdgcn_perm(x3, x2, 0x0C0C0400u);  // [x2.b0, x3.b0, 0, 0]
  return __builtin_amdgcn_perm(b, a, 0x05040100u);                // [a.b0, a.b1, b.b0, b.b1]
}

// ---------------------------------------------------------------------------
// GEMM operand decode (E2M1 code x E4M3 block scale -> FP16, exact)
// ---------------------------------------------------------------------------

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

// Two E4M3 scale bytes (bits 0..7 and 8..15 of w) -> two FP16 values S * 2^-8
// in one dword: an E4M3 code shifted left by 7 and read as FP16 is its value
// times 2^-8 (exponent fields line up; subnormal codes become FP16
// subnormals).  The converter's scale of 256 below supplies the missing 2^8.
__device__ __forceinline__ half2_t scale_pair_lo(uint32_t w) {
  return __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0u, w, 0x0C010C00u) << 7);
}

// Eight E2M1 codes times (S * 2^-8): the converter at scale 2^8 (exact, a
// power of two) gives code * 256, and one packed multiply per pair gives
// code * S, exact in FP16 (at most 6 significant bits, at least 2^-10).
// tests/test_hw_converters.py checks every code against every scale byte.
__device__ __forceinline__ half8_t decode8_s256(uint32_t codes, _Float16 s) {
  const half2_t s2 = {s, s};
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 0) * s2;
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 1) * s2;
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 2) * s2;
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 3) * s2;
  return half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Two FP32 values -> two BF16 (round to nearest even) in one dword, the
// first in the low half: gfx950's v_cvt_pk_bf16_f32 (the GEMM epilogue's
// convert; tests/test_hw_converters.py sweeps every FP32 pattern through it).
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  typedef float float2_v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  const float2_v y2 = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(y2, bf16x2_v));
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11)
// ---------------------------------------------------------------------------

struct u32x4 {
  uint32_t x, y, z, w;
};

// a ^ b ^ k in one VALU instruction (gfx950's three-input bit operation,
// truth table 0x96); k is uniform over the wavefront (a key word), so it is
// taken from a scalar register.
__device__ __forceinline__ uint32_t xor3_key(uint32_t a, uint32_t b, uint32_t k) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
  return r;
}

// Each round's two 32 x 32 -> 64-bit products are written as one 64-bit
// multiply each, which the compiler emits as a single v_mad_u64_u32 (the
// high and low words at once) instead of a mul_lo / mul_hi pair.  The key
// must be uniform over the wavefront (it is a kernel argument here).
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x, p1 = (uint64_t)0xCD9E8D57u * c.z;
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    c = u32x4{xor3_key(hi1, c.y, k0), lo1, xor3_key(hi0, c.w, k1), lo0};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// The 16 signs of the random Hadamard transform as a bit mask (bit j set:
// s_j = -1): word 0 of the block at counter (0, 0, ~0, 0) under the seed.
__device__ __forceinline__ uint32_t rht_sign_mask(uint64_t seed) {
  return philox4x32_10(u32x4{0u, 0u, 0xFFFFFFFFu, 0u}, (uint32_t)seed, (uint32_t)(seed >> 32)).x &
         0xFFFFu;
}

// The eight 16-bit stochastic-rounding words of logical elements 8g..8g+7.
__device__ __forceinline__ u32x4 sr_block(uint64_t g, uint32_t stream, uint64_t seed) {
  return philox4x32_10(u32x4{(uint32_t)g, (uint32_t)(g >> 32), stream, 0u}, (uint32_t)seed,
                       (uint32_t)(seed >> 32));
}


// ---------------------------------------------------------------------------
// Lane-pair exchange
// ---------------------------------------------------------------------------

// The value of the other lane of the pair (2k, 2k + 1): a DPP quad
// permutation [1, 0, 3, 2], i.e. a VALU move with no LDS traffic.
__device__ __forceinline__ uint32_t lane_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ float lane_xor1(float v) { return __uint_as_float(lane_xor1(__float_as_uint(v))); }

// ---------------------------------------------------------------------------
// Random Hadamard transform on 16 values held by one lane
// ---------------------------------------------------------------------------

// v <- H16 diag(s) v; signs flip by XOR of the sign bit (exact), the
// butterflies run with span 1, 2, 4, 8 in that order in FP32.
__device__ __forceinline__ void rht16_unscaled(float (&v)[16], uint32_t mask) {
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = __uint_as_float(__float_as_uint(v[j]) ^ (((mask >> j) & 1u) << 31));
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      const float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
}

// v <- (1/4) H16 diag(s) v: the butterflies, then the product by 1/4 of each
// value (rounded, which matters only for subnormal results).
__device__ __forceinline__ void rht16(float (&v)[16], uint32_t mask) {
  rht16_unscaled(v, mask);
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = v[j] * 0.25f;
}

// max |v'| over a block of v' = fl(w / 4), as FP32 bits, from the maximum of
// |w| (bits m): rounding is monotone, so fl(max|w| / 4) = max fl(|w| / 4).
__device__ __forceinline__ uint32_t quarter_max_bits(uint32_t m) {
  return __float_as_uint(__uint_as_float(m) * 0.25f);
}

// ---------------------------------------------------------------------------
// Reductions over |x| as unsigned bit patterns (NaN patterns sort above all
// finite values, so a NaN input poisons the maximum).
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t abs_bits(float f) { return __float_as_uint(f) & 0x7FFFFFFFu; }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
  return v;
}

}  // namespace nvfp4
