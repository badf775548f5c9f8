// Device helpers shared by the libmxfp4 kernels (gfx950 / CDNA4).
//
// Format facts used here ("MXFP4", AI Wiki, §Format specification and
// §Conversion rules): E2M1 codes carry magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 in
// code order 0..7 with the sign in bit 3; E8M0 scale byte s means 2^(s-127)
// and 0xFF is NaN; the reference shared exponent is floor(log2 amax) - 2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// ---------------------------------------------------------------- bit helpers
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return ((b >> 16) | 0x40u) & 0xFFFFu;
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Cross-lane reads inside a quad of 4 lanes (DPP quad_perm, one VALU op).
__device__ __forceinline__ uint32_t quad_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);   // [1,0,3,2]
}
__device__ __forceinline__ uint32_t quad_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);   // [2,3,0,1]
}
__device__ __forceinline__ float quad_xor1f(float v) { return __uint_as_float(quad_xor1(__float_as_uint(v))); }
__device__ __forceinline__ float quad_xor2f(float v) { return __uint_as_float(quad_xor2(__float_as_uint(v))); }

// ---------------------------------------------------------------- Philox4x32-10
// Salmon et al., SC'11: ten rounds of two 32x32->64 multiplies, key bumped by
// the Weyl constants between rounds.
struct u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
    // three-way XORs as one V_BITOP3_B32 each (truth table 0x96)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return {c0, c1, c2, c3};
}

// The stochastic-rounding draws of Philox call q, which serves elements
// 8q..8q+7 of the output in row-major [rows_out, K] order: element t takes the
// 16-bit half (t & 1) of word w[t >> 1] (low half first).
__device__ __forceinline__ void sr_words(uint64_t q, uint64_t seed, uint64_t offset, uint32_t w[4]) {
  const u32x4 v = philox4x32_10((uint32_t)q, (uint32_t)(q >> 32), (uint32_t)offset,
                                (uint32_t)(offset >> 32), (uint32_t)seed, (uint32_t)(seed >> 32));
  w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
}

// ---------------------------------------------------------------- scale
// Scale byte from the largest |y| of a block given as float32 bits with the
// sign cleared: NaN/Inf -> 0xFF; otherwise biased_exponent(amax) - 2 clamped
// at 0 (this is floor(log2 amax) - 2 + 127, and covers zero and subnormal
// amax, whose floor(log2) is below -126).
__device__ __forceinline__ uint32_t scale_code_from_absmax_bits(uint32_t m) {
  if (m >= 0x7F800000u) return 0xFFu;
  const int be = (int)(m >> 23);
  return (uint32_t)(be > 2 ? be - 2 : 0);
}

// Round-up rule: the smallest power of two X with amax / X <= 6, i.e. the
// exponent ceil(log2(amax / 6)) = floor(log2 amax) - 2 + (mantissa > 1.5),
// clamped at 0 (zero and subnormal amax, and amax below 1.5 * 2^-125, give
// byte 0); NaN/Inf -> 0xFF.
__device__ __forceinline__ uint32_t scale_code_round_up(uint32_t m) {
  if (m >= 0x7F800000u) return 0xFFu;
  const int c = (int)(m >> 23) - 2 + (int)((m & 0x7FFFFFu) > 0x400000u);
  return (uint32_t)(c > 0 ? c : 0);
}

// 2^-(s-127) as float32 for a finite scale byte s <= 253 (always a normal).
__device__ __forceinline__ float inv_scale_from_code(uint32_t s) {
  return __uint_as_float((254u - s) << 23);
}

// ---------------------------------------------------------------- E2M1 rounding
// v is already divided by the block scale (|v| < 8 for a finite block).
// Integer form of round-to-nearest-even onto {0,.5,1,1.5,2,3,4,6}:
//  |v| >= 1: the E2M1 grid is float32 with one mantissa bit, so round the
//            float32 bits at bit 22 (ties to an even bit 22) and read the code
//            from the exponent and that bit; codes above 7 saturate to 7.
//  |v| <  1: step 0.5; (0.25, 0.75) -> 0.5, [0.75, 1) -> 1.0, ties 0.25 -> 0
//            and 0.75 -> 1.0 (both even mantissa).
__device__ __forceinline__ uint32_t e2m1_rne(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sgn = (b >> 28) & 8u;
  const uint32_t a = b & 0x7FFFFFFFu;
  uint32_t idx;
  if (a >= 0x3F800000u) {
    const uint32_t t = (a + 0x1FFFFFu + ((a >> 22) & 1u)) >> 22;
    idx = min(t - 252u, 7u);
  } else {
    idx = (uint32_t)(a > 0x3E800000u) + (uint32_t)(a >= 0x3F400000u);
  }
  return sgn | idx;
}

// Stochastic rounding with a 16-bit draw r: the magnitude rounds up from the
// lower grid point lo to the upper one iff r < f * 2^16, where f is the exact
// fraction of the way from lo to the next grid point; |v| >= 6 saturates.
//  |v| >= 1   : lo from the truncated bits, f * 2^22 = the 22 bits below bit 22.
//  .5 <= |v| < 1: lo = .5, f * 2^23 = the 23 mantissa bits.
//  |v| < .5   : lo = 0, f = 2|v|; compare in float32 (exact, power-of-two scaling).
__device__ __forceinline__ uint32_t e2m1_sr(float v, uint32_t r) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sgn = (b >> 28) & 8u;
  const uint32_t a = b & 0x7FFFFFFFu;
  uint32_t idx;
  if (a >= 0x3F800000u) {
    const uint32_t lo = (a >> 22) - 252u;
    idx = min(lo + (uint32_t)((r << 6) < (a & 0x3FFFFFu)), 7u);
  } else if (a >= 0x3F000000u) {
    idx = 1u + (uint32_t)((r << 7) < (a & 0x7FFFFFu));
  } else {
    idx = (uint32_t)((float)r < __uint_as_float(a) * 131072.0f);
  }
  return sgn | idx;
}

// E2M1 magnitude of a 4-bit code as float32 (sign applied).
__device__ __forceinline__ float e2m1_value(uint32_t code) {
  const uint32_t m = code & 7u;
  uint32_t bits = (m >= 2u) ? ((((m >> 1) + 126u) << 23) | ((m & 1u) << 22))
                            : (m == 1u ? 0x3F000000u : 0u);
  return __uint_as_float(bits | ((code & 8u) << 28));
}

// 2^(s-127) as float32 for a scale byte (s = 0 gives the subnormal 2^-127,
// s = 0xFF gives NaN).
__device__ __forceinline__ float scale_value(uint32_t s) {
  if (s == 0xFFu) return __uint_as_float(0x7FC00000u);
  return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);
}

// Hardware RNE conversion: V_CVT_SCALEF32_PK_FP4_F32 writes two E2M1 codes
// (x0 in the low nibble) into byte `sel` of `old`, computing
// RNE_fp4(RNE_fp32(x / scale)) with saturation to +-6 and the sign of zero
// kept.  For a power-of-two scale this is exactly the conversion above
// (verified exhaustively over all float32 inputs for scales 2^-126 .. 2^125 by
// the probe tests), so the quantizer hands it the block scale directly.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_pk_fp4(uint32_t old, float x0, float x1, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, x0, x1, scale, SEL);
}

// 8 values -> one 32-bit word of codes (value i in nibble i), RNE.
__device__ __forceinline__ uint32_t pack8_rne(const float x[8], float scale) {
  uint32_t w = 0;
  w = cvt_pk_fp4<0>(w, x[0], x[1], scale);
  w = cvt_pk_fp4<1>(w, x[2], x[3], scale);
  w = cvt_pk_fp4<2>(w, x[4], x[5], scale);
  w = cvt_pk_fp4<3>(w, x[6], x[7], scale);
  return w;
}

// Hardware stochastic rounding, equal to e2m1_sr.  V_CVT_SCALEF32_SR_PK_FP4_F32
// puts x / scale in fixed point with 22 bits below the E2M1 step, dropping
// finer bits, adds the top 22 bits of its random operand (bits 31..10 for
// element 0) and truncates; it saturates at +-6 and keeps the sign.  Writing
// F for the fraction f * 2^22 of e2m1_sr, it rounds up iff
// floor(F) + R22 >= 2^22.  For |v| >= 1 the E2M1 step spans 22 mantissa bits,
// so F is already an integer; below 1 (step 0.5) a float32 can carry finer
// bits.  So the element goes in as t = sign(v) ceil(|v| 2^23) with scale 2^23:
// t / 2^23 is exact (|t| <= 2^26), F becomes ceil(F) and is unchanged for
// |v| >= 1, and with R22 = (~r) 2^6 + 63 the hardware rounds up iff
// ceil(F) > 64 r, i.e. iff r < f 2^16.  Each element's code comes from its
// own convert: the two elements of one instruction read overlapping random
// bits (element 1 reads bits 30..9), while e2m1_sr draws independent 16-bit
// halves.  The probe tests compare this with e2m1_sr for every
// float32 |v| < 8 at the draws on both sides of the rounding threshold.
__device__ __forceinline__ float sr_fixed_point(float v) {
  return __uint_as_float((__float_as_uint(__builtin_ceilf(__builtin_fabsf(v) * 8388608.0f)) & 0x7FFFFFFFu) |
                         (__float_as_uint(v) & 0x80000000u));
}

// Codes of v0 (low nibble) and v1 (high nibble) in bits 7..0 of the result;
// bits 31..8 are undefined.  w carries the draws: r0 = w & 0xFFFF,
// r1 = w >> 16.  Both converts take the pair (t0, t1); the first is given the
// random field of element 0 and supplies the low nibble, the second that of
// element 1 and supplies the high nibble.  (The compiler does not treat the
// builtin's `old` operand as an input, so only byte 0 of a result is read.)
__device__ __forceinline__ uint32_t cvt_sr_pair(float v0, float v1, uint32_t w) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  const v2f t = {sr_fixed_point(v0), sr_fixed_point(v1)};
  const uint32_t nw = ~w;
  const uint32_t R0 = (nw << 16) | 0xFFFFu;  // bits 31..10 read by element 0: ~r0, then ones
  const uint32_t R1 = (nw >> 1) | 0x7FFFu;   // bits 30..9 read by element 1: ~r1, then ones
  const uint32_t c0 = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, t, R0, 8388608.0f, 0);
  const uint32_t c1 = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, t, R1, 8388608.0f, 0);
  return (c0 & 0x0Fu) | (c1 & ~0x0Fu);   // one V_BFI_B32
}

// 8-bit draws as 16-bit ones: bytes 2H and 2H + 1 of a Philox word w, the
// draws of two consecutive elements, as the word (b1 << 24) | (b0 << 8)
// that pack8_sr reads (draw 256 b in each 16-bit half; V_PERM_B32 selector
// 0x0C gives a zero byte).
template <int H>
__device__ __forceinline__ uint32_t sr8_pair(uint32_t w) {
  return __builtin_amdgcn_perm(w, w, H ? 0x030C020Cu : 0x010C000Cu);
}

// 8 values (already divided by the block scale) -> one word of SR codes;
// value 2j uses the low half of w[j], value 2j+1 the high half.
__device__ __forceinline__ uint32_t pack8_sr(const float v[8], const uint32_t w[4]) {
  const uint32_t p0 = cvt_sr_pair(v[0], v[1], w[0]);
  const uint32_t p1 = cvt_sr_pair(v[2], v[3], w[1]);
  const uint32_t p2 = cvt_sr_pair(v[4], v[5], w[2]);
  const uint32_t p3 = cvt_sr_pair(v[6], v[7], w[3]);
  // byte 0 of each pair result -> bytes 0..3 (V_PERM_B32: selector 0..3 picks
  // a byte of the second operand, 4..7 of the first, 0x0C gives zero)
  return __builtin_amdgcn_perm(p1, p0, 0x0C0C0400u) | __builtin_amdgcn_perm(p3, p2, 0x04000C0Cu);
}

// Block scale 2^(s-127) as the float32 the conversion divides by.  The lowest
// byte s = 0 (2^-127, a float32 subnormal) is avoided by the callers: they
// multiply by 2^127 themselves and convert with scale 1.0.
__device__ __forceinline__ float scale_f32_normal(uint32_t s) { return __uint_as_float(s << 23); }

// ---------------------------------------------------------------- Hadamard
// Radix-2 butterflies of the 32-point fast Walsh-Hadamard transform in
// Sylvester order: stage h maps (x_i, x_{i+h}) -> (x_i + x_{i+h}, x_i - x_{i+h})
// for i & h == 0.  Stages 1, 2, 4 act inside 8 consecutive elements.
__device__ __forceinline__ void fwht8_inlane(float x[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
}

// Stages 8 and 16 when lane j of a quad holds elements 8j..8j+7 of the block:
// the partner of element i is in lane j ^ 1 (h = 8) or j ^ 2 (h = 16); the lane
// holding the lower index keeps the sum, the other keeps lower - upper.
//
// Fast form: every lane computes x + k * partner with k = +1 (lower lane) or
// -1 (upper lane) in one fused multiply-add, which is exactly the rounded sum
// or difference; the upper lane then holds the negated value, and the signs
// are carried to the end: the returned factor (+-1) times the stored value is
// the true transform value.
__device__ __forceinline__ float fwht_cross_quad_signed(float x[8], uint32_t quad_lane) {
  const float k8 = (quad_lane & 1u) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = __builtin_fmaf(quad_xor1f(x[i]), k8, x[i]);
  const float k16 = (quad_lane & 2u) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = __builtin_fmaf(quad_xor2f(x[i]), k16, x[i]);
  return k8 * k16;
}

__device__ __forceinline__ void fwht_cross_quad(float x[8], uint32_t quad_lane) {
  const bool up8 = quad_lane & 1u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = quad_xor1f(x[i]);
    x[i] = up8 ? (p - x[i]) : (x[i] + p);
  }
  const bool up16 = quad_lane & 2u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = quad_xor2f(x[i]);
    x[i] = up16 ? (p - x[i]) : (x[i] + p);
  }
}

// All five stages for a block held by one lane.
__device__ __forceinline__ void fwht32_inlane(float x[32]) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
}

constexpr uint32_t kRhtCBits = 0x3E3504F3u;   // float32(1/sqrt(32))

// ---------------------------------------------------------------- other MX element types
// FP8 (E4M3, E5M2) and FP6 (E2M3, E3M2) elements of MXFP8 / MXFP6 ("MXFP4",
// AI Wiki, §Place in the MX family), with the OCP element definitions: E
// exponent bits of bias 2^(E-1)-1, M mantissa bits, subnormals at exponent
// field 0; E4M3's S.1111.111 is NaN (largest normal 448), E5M2's top exponent
// is Inf/NaN (largest normal 57344), FP6 has no Inf/NaN (largest normals 7.5
// and 28).  ELEM is the mx_elem value (1..4); E2M1 (0) keeps the code above.
template <int ELEM>
struct ElemT;
template <>
struct ElemT<1> {   // E4M3
  static constexpr int E = 4, M = 3, BIAS = 7, MAXCODE = 0x7E, EMAX = 8, BITS = 8, MFMA = 0;
  static constexpr uint32_t MAXBITS = 0x43E00000u;   // 448 = 1.75 * 2^8
};
template <>
struct ElemT<2> {   // E5M2
  static constexpr int E = 5, M = 2, BIAS = 15, MAXCODE = 0x7B, EMAX = 15, BITS = 8, MFMA = 1;
  static constexpr uint32_t MAXBITS = 0x47600000u;   // 57344 = 1.75 * 2^15
};
template <>
struct ElemT<3> {   // E2M3
  static constexpr int E = 2, M = 3, BIAS = 1, MAXCODE = 0x1F, EMAX = 2, BITS = 6, MFMA = 2;
  static constexpr uint32_t MAXBITS = 0x40F00000u;   // 7.5 = 1.875 * 2^2
};
template <>
struct ElemT<4> {   // E3M2
  static constexpr int E = 3, M = 2, BIAS = 3, MAXCODE = 0x1F, EMAX = 4, BITS = 6, MFMA = 3;
  static constexpr uint32_t MAXBITS = 0x41E00000u;   // 28 = 1.75 * 2^4
};

// Bits per element of mx_elem ELEM (0 is E2M1).
template <int ELEM>
constexpr int elem_bits() {
  if constexpr (ELEM == 0) return 4;
  else return ElemT<ELEM>::BITS;
}

// Scale byte of a block whose largest magnitude has float32 bits m (sign
// cleared): the reference rule floor(log2 amax) - EMAX, or (ROUND_UP) the
// smallest exponent e with amax <= largest normal * 2^e; clamped at 0; NaN or
// Inf give 0xFF.
template <int ELEM>
__device__ __forceinline__ uint32_t elem_scale_code(uint32_t m, bool round_up) {
  using T = ElemT<ELEM>;
  if (m >= 0x7F800000u) return 0xFFu;
  const int c = (int)(m >> 23) - T::EMAX + (round_up ? (int)((m & 0x7FFFFFu) > (T::MAXBITS & 0x7FFFFFu)) : 0);
  return (uint32_t)(c > 0 ? c : 0);
}

// Magnitude code of a = |v| (v already divided by the block scale, finite):
// with Ec the binade of a (at least the subnormal binade 1 - BIAS), the grid
// spacing is 2^(Ec - M) and t = a * 2^(M - Ec) is exact; the code is
// ((Ec + BIAS - 1) << M) + round(t), continuous across binades, and saturates
// at the largest normal.  RNE rounds t to even (an even t is an even code);
// SR rounds up iff the 16 random bits r are below frac(t) * 2^16.
template <int ELEM, bool SR>
__device__ __forceinline__ uint32_t elem_mag_code(float a, uint32_t r16) {
  using T = ElemT<ELEM>;
  const uint32_t ab = __float_as_uint(a);
  if (ab >= T::MAXBITS) return T::MAXCODE;
  const int ev = (int)(ab >> 23) - 127;
  const int ec = ev > 1 - T::BIAS ? ev : 1 - T::BIAS;
  const float t = a * __uint_as_float((uint32_t)(127 + T::M - ec) << 23);
  uint32_t n;
  if (SR) {
    const float fl = __builtin_floorf(t);
    n = (uint32_t)fl + (uint32_t)((float)r16 < (t - fl) * 65536.0f);
  } else {
    n = (uint32_t)__builtin_rintf(t);
  }
  const uint32_t code = ((uint32_t)(ec + T::BIAS - 1) << T::M) + n;
  return code < (uint32_t)T::MAXCODE ? code : (uint32_t)T::MAXCODE;
}

template <int ELEM, bool SR>
__device__ __forceinline__ uint32_t elem_code(float v, uint32_t r16) {
  using T = ElemT<ELEM>;
  return elem_mag_code<ELEM, SR>(__builtin_fabsf(v), r16) | ((__float_as_uint(v) >> 31) << (T::E + T::M));
}

// Hardware RNE conversion for the FP8 / FP6 element types.
// V_CVT_SCALEF32_PK_FP8_F32 / _PK_BF8_F32 (E4M3 / E5M2, two values) and
// V_CVT_SCALEF32_2XPK16_FP6_F32 / _BF6_F32 (E2M3 / E3M2, 32 values) round
// x / scale to nearest even.  The FP8 forms do not saturate: from the midpoint
// above the largest normal they return the NaN / Inf code (the probe tests saw
// E4M3 0x7F for x / scale = 481.8).  Clamping x to +-(largest normal * scale)
// first is exact for a power-of-two scale and makes the result equal to
// elem_code<ELEM, false>(x / scale) for every finite float32 x; the probe
// tests check these helpers against elem_code over all finite float32 inputs
// at several scales.  lim is largest normal * scale (Inf when that overflows:
// then no finite quotient reaches the largest normal).
__device__ __forceinline__ float elem_clamp(float x, float lim) { return __builtin_amdgcn_fmed3f(x, -lim, lim); }

// Four values -> one word of FP8 codes, value i in byte i.
template <int ELEM>
__device__ __forceinline__ uint32_t pack4_fp8(const float x[4], float scale, float lim) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  v2s w = {0, 0};
  const float a0 = elem_clamp(x[0], lim), a1 = elem_clamp(x[1], lim);
  const float a2 = elem_clamp(x[2], lim), a3 = elem_clamp(x[3], lim);
  if constexpr (ELEM == 1) {
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, a0, a1, scale, false);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, a2, a3, scale, true);
  } else {
    w = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(w, a0, a1, scale, false);
    w = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(w, a2, a3, scale, true);
  }
  return __builtin_bit_cast(uint32_t, w);
}

// 32 values -> 6 words of FP6 codes, value e at bits 6e .. 6e+5.  The
// instruction interleaves its two 16-value sources (code 2i from the first
// source's value i, code 2i+1 from the second's; seen in the probe tests), so
// the even values go in the first source and the odd values in the second.
template <int ELEM>
__device__ __forceinline__ void pack32_fp6(const float x[32], float scale, float lim, uint32_t out[6]) {
  typedef float v16 __attribute__((ext_vector_type(16)));
  typedef int v6 __attribute__((ext_vector_type(6)));
  v16 a, b;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    a[i] = elem_clamp(x[2 * i], lim);
    b[i] = elem_clamp(x[2 * i + 1], lim);
  }
  v6 p;
  if constexpr (ELEM == 3)
    p = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, scale);
  else
    p = __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(a, b, scale);
#pragma unroll
  for (int j = 0; j < 6; ++j) out[j] = (uint32_t)p[j];
}

// Value of a code (NaN and Inf codes decode as such).
template <int ELEM>
__device__ __forceinline__ float elem_value(uint32_t c) {
  using T = ElemT<ELEM>;
  const uint32_t e = (c >> T::M) & ((1u << T::E) - 1u), f = c & ((1u << T::M) - 1u);
  float mag = e == 0 ? (float)f * __uint_as_float((uint32_t)(127 + 1 - T::BIAS - T::M) << 23)
                     : (float)((1u << T::M) | f) * __uint_as_float((uint32_t)(127 + (int)e - T::BIAS - T::M) << 23);
  if (ELEM == 1 && e == 15u && f == 7u) mag = __builtin_nanf("");
  if (ELEM == 2 && e == 31u) mag = f == 0 ? __builtin_inff() : __builtin_nanf("");
  return (c >> (T::E + T::M)) & 1u ? -mag : mag;
}

// ------------------------------------------------------ the MXFP4 block step
// Quantize one block held in registers (x already sign-flipped when RHT).
// Returns the scale byte and writes the 16 code bytes to `packed`.
// With TWO_D the amax is taken over the 32 lanes of the half-wave as well
// (one lane per column of a 32x32 tile; all 32 lanes must be active).
// scale_mode (wave-uniform): 0 the reference rule floor(log2 amax) - 2; 1 the
// round-up rule; 2 the reference rule's scale with every element multiplied by
// 0.75 (one float32 multiply) before the division, so nothing clips.
template <bool RHT, int SR, bool TWO_D = false>
__device__ __forceinline__ uint32_t quantize_block32(float x[32], uint32_t packed[4], uint64_t p0,
                                                     uint64_t seed, uint64_t offset, int scale_mode) {
  const float c = __uint_as_float(kRhtCBits);
  if (RHT) fwht32_inlane(x);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = max(m, __float_as_uint(x[i]) & 0x7FFFFFFFu);
  // multiplying by a positive constant commutes with the max (rounding is monotone)
  if (RHT) {
    m = __float_as_uint(c * __uint_as_float(m));      // max |c t_i| = c max |t_i|
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = c * x[i];
  }
  if (TWO_D) {
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d, 32));
  }
  const uint32_t s = scale_mode == 1 ? scale_code_round_up(m) : scale_code_from_absmax_bits(m);
  packed[0] = packed[1] = packed[2] = packed[3] = 0u;
  if (s == 0xFFu) return s;
  if (scale_mode == 2) {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = 0.75f * x[i];
  }
  if (SR) {
    const float inv = inv_scale_from_code(s);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t w[4];
      if constexpr (SR == 2) {
        // 8-bit draws: one Philox call per 16 elements, element i of the call
        // taking byte (i & 3) of word i >> 2; each byte b goes in as the
        // 16-bit draw 256 b, with which the 16-bit rule rounds up exactly
        // when b < 256 f
        uint32_t W[4];
        sr_words((p0 >> 4) + (g >> 1), seed, offset, W);
        const uint32_t w0 = W[2 * (g & 1)], w1 = W[2 * (g & 1) + 1];
        w[0] = sr8_pair<0>(w0);
        w[1] = sr8_pair<1>(w0);
        w[2] = sr8_pair<0>(w1);
        w[3] = sr8_pair<1>(w1);
      } else {
        sr_words((p0 >> 3) + g, seed, offset, w);
      }
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = x[8 * g + i] * inv;
      packed[g] = pack8_sr(v, w);
    }
  } else {
    float sc = scale_f32_normal(s);
    if (s == 0u) {
      // scale 2^-127 is a float32 subnormal: multiply by 2^127 instead and
      // convert at scale 1 (the same single rounding)
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = x[i] * __uint_as_float(0x7F000000u);
      sc = 1.0f;
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) packed[g] = pack8_rne(x + 8 * g, sc);
  }
  return s;
}

}  // namespace mx
