// codec_math.h -- bit-level encoders and decoders of the element and scale formats, shared by
// the host codec and the GPU codec kernels (both sides run exactly this arithmetic, so the two
// are bit-identical by construction).
//
// Element formats (named by "Optimize custom machine learning operations with Metal tensors",
// quantized data types and MXFP8 tensor type, and by the TensorOps notes' dtype matrix: fp8, fp4,
// MX scaling formats; bit layouts from the OCP Microscaling v1.0 spec):
//   E4M3 "FN": s.eeee.mmm, bias 7, exponent 0 subnormal (m * 2^-9), s.1111.111 NaN, max 448.
//   E5M2:      s.eeeee.mm, bias 15, exponent 0 subnormal (m * 2^-16), s.11111.00 Inf,
//              s.11111.mm (m != 0) NaN, max 57344.
//   E2M3:      s.ee.mmm (6 bits), bias 1, exponent 0 subnormal (m * 2^-3), max 7.5, no NaN/Inf.
//   E3M2:      s.eee.mm (6 bits), bias 3, exponent 0 subnormal (m * 2^-4), max 28, no NaN/Inf.
//              FP6 rows pack element j into bits 6j..6j+5 of a little-endian bit stream.
//   E2M1:      s.ee.m, bias 1, exponent 0 subnormal (m * 0.5), max 6, no NaN.
//   E8M0:      2^(e-127), 0xFF = NaN.
// Encoding is round-to-nearest, ties to the even code, with saturation to the largest finite
// value. It works on the integer significand of the fp32 input and an exponent offset, so no
// intermediate fp32 product can be rounded or flushed.
#pragma once
#include "common.h"

namespace mx {

MX_HD uint32_t fbits(float f) { return __builtin_bit_cast(uint32_t, f); }
MX_HD float bitsf(uint32_t u) { return __builtin_bit_cast(float, u); }

// floor(log2 a) for the bit pattern a of a finite, positive fp32 value (subnormals included).
MX_HD int ilog2_bits(uint32_t a) {
  uint32_t ef = a >> 23;
  return ef ? (int)ef - 127 : (31 - __builtin_clz(a)) - 149;
}

// 24-bit significand with the leading one at bit 23, for a finite positive fp32 bit pattern.
MX_HD uint32_t norm_sig(uint32_t a) {
  if (a >> 23) return (a & 0x7FFFFFu) | 0x800000u;
  return a << (23 - (31 - __builtin_clz(a)));
}

// Round sig / 2^sh to the nearest integer, ties to even (sig < 2^25, sh >= 1).
MX_HD uint32_t rne_shift(uint32_t sig, int sh) {
  if (sh >= 26) return 0u;
  uint32_t r = sig >> sh, rem = sig & ((1u << sh) - 1u), half = 1u << (sh - 1);
  return r + (uint32_t)((rem > half) | ((rem == half) & (r & 1u)));
}

// E4M3 magnitude code (0..0x7E) of |x| * 2^t, a = bits of |x| (finite).
MX_HD uint32_t e4m3_mag(uint32_t a, int t) {
  if (a == 0u) return 0u;
  int ev = ilog2_bits(a) + t;                    // |x| 2^t lies in [2^ev, 2^(ev+1))
  uint32_t sig = norm_sig(a);
  if (ev > 8 || (ev == 8 && sig >= 0xE00000u)) return 0x7Eu;  // >= 448: saturate
  if (ev >= -6) {                                // normal E4M3: 3 fraction bits
    uint32_t r = rne_shift(sig, 20);
    int e = ev;
    if (r == 16u) { r = 8u; e++; }
    return ((uint32_t)(e + 7) << 3) | (r - 8u);
  }
  return rne_shift(sig, 14 - ev);                // subnormal E4M3: multiples of 2^-9 (0..8)
}

// E5M2 magnitude code (0..0x7B) of |x| * 2^t, a = bits of |x| (finite).
MX_HD uint32_t e5m2_mag(uint32_t a, int t) {
  if (a == 0u) return 0u;
  int ev = ilog2_bits(a) + t;
  uint32_t sig = norm_sig(a);
  if (ev > 15 || (ev == 15 && sig >= 0xE00000u)) return 0x7Bu;  // >= 57344: saturate
  if (ev >= -14) {                               // normal E5M2: 2 fraction bits
    uint32_t r = rne_shift(sig, 21);
    int e = ev;
    if (r == 8u) { r = 4u; e++; }
    return ((uint32_t)(e + 15) << 2) | (r - 4u);
  }
  return rne_shift(sig, 7 - ev);                 // subnormal E5M2: multiples of 2^-16 (0..4)
}

// E2M3 magnitude code (0..31) of |x| * 2^t.
MX_HD uint32_t e2m3_mag(uint32_t a, int t) {
  if (a == 0u) return 0u;
  int ev = ilog2_bits(a) + t;
  uint32_t sig = norm_sig(a);
  if (ev > 2 || (ev == 2 && sig >= 0xF00000u)) return 31u;     // >= 7.5: saturate
  if (ev >= 0) {                                 // normal E2M3: 3 fraction bits
    uint32_t r = rne_shift(sig, 20);
    int e = ev;
    if (r == 16u) { r = 8u; e++; }
    return ((uint32_t)(e + 1) << 3) | (r - 8u);
  }
  return rne_shift(sig, 20 - ev);                // subnormal E2M3: multiples of 2^-3 (0..8)
}

// E3M2 magnitude code (0..31) of |x| * 2^t.
MX_HD uint32_t e3m2_mag(uint32_t a, int t) {
  if (a == 0u) return 0u;
  int ev = ilog2_bits(a) + t;
  uint32_t sig = norm_sig(a);
  if (ev > 4 || (ev == 4 && sig >= 0xE00000u)) return 31u;     // >= 28: saturate
  if (ev >= -2) {                                // normal E3M2: 2 fraction bits
    uint32_t r = rne_shift(sig, 21);
    int e = ev;
    if (r == 8u) { r = 4u; e++; }
    return ((uint32_t)(e + 3) << 2) | (r - 4u);
  }
  return rne_shift(sig, 19 - ev);                // subnormal E3M2: multiples of 2^-4 (0..4)
}

// E2M1 magnitude code (0..7) of |x| * 2^t.
MX_HD uint32_t e2m1_mag(uint32_t a, int t) {
  if (a == 0u) return 0u;
  int ev = ilog2_bits(a) + t;
  uint32_t sig = norm_sig(a);
  if (ev > 2 || (ev == 2 && sig >= 0xC00000u)) return 7u;     // >= 6: saturate
  if (ev >= 0) {                                 // normal E2M1: 1 fraction bit
    uint32_t r = rne_shift(sig, 22);
    int e = ev;
    if (r == 4u) { r = 2u; e++; }
    return ((uint32_t)(e + 1) << 1) | (r - 2u);
  }
  return rne_shift(sig, 22 - ev);                // subnormal E2M1: multiples of 0.5 (0..2)
}

// Element formats by their mx_format codes: E4M3 = 0, E5M2 = 1, E2M3 = 2, E3M2 = 3, E2M1 = 4.
constexpr bool is_byte_fmt(int fmt) { return fmt == MX_E4M3 || fmt == MX_E5M2; }
constexpr bool is_fp6_fmt(int fmt) { return fmt == MX_E2M3 || fmt == MX_E3M2; }

// Element code of x * 2^t with the sign of x kept, in format fmt.
MX_HD uint32_t enc_elem_fmt(int fmt, float x, int t) {
  uint32_t u = fbits(x), a = u & 0x7FFFFFFFu, s = u >> 31;
  if (fmt == MX_E4M3) return (s << 7) | e4m3_mag(a, t);
  if (fmt == MX_E5M2) return (s << 7) | e5m2_mag(a, t);
  if (fmt == MX_E2M3) return (s << 5) | e2m3_mag(a, t);
  if (fmt == MX_E3M2) return (s << 5) | e3m2_mag(a, t);
  return (s << 3) | e2m1_mag(a, t);
}

// E8M0 scale code of a block from the bit pattern of its amax (finite, >= 0):
// clamp(floor(log2 amax) - emax + 127, 0, 254), 0 when amax = 0.
MX_HD uint32_t scale_code(uint32_t amax_bits, int emax) {
  if (amax_bits == 0u) return 0u;
  int E = ilog2_bits(amax_bits) - emax + 127;
  return (uint32_t)(E < 0 ? 0 : (E > 254 ? 254 : E));
}

// Decoders to fp32 (exact).
MX_HD float dec_e8m0(uint32_t e) {
  e &= 0xFFu;
  if (e == 0xFFu) return bitsf(0x7FC00000u);
  return e ? bitsf(e << 23) : bitsf(0x00400000u);  // e = 0 is 2^-127, an fp32 subnormal
}

MX_HD float dec_e4m3(uint32_t b) {
  uint32_t s = (b & 0x80u) << 24, e = (b >> 3) & 15u, m = b & 7u;
  if ((b & 0x7Fu) == 0x7Fu) return bitsf(0x7FC00000u | s);
  if (e) return bitsf(s | ((e + 120u) << 23) | (m << 20));
  return bitsf(s | fbits((float)m * 0.001953125f));  // m * 2^-9, exact
}

MX_HD float dec_e5m2(uint32_t b) {
  uint32_t s = (b & 0x80u) << 24, e = (b >> 2) & 31u, m = b & 3u;
  if (e == 31u) return bitsf(s | (m ? 0x7FC00000u : 0x7F800000u));
  if (e) return bitsf(s | ((e + 112u) << 23) | (m << 21));
  return bitsf(s | fbits((float)m * 1.52587890625e-05f));  // m * 2^-16, exact
}

MX_HD float dec_e2m3(uint32_t c) {
  uint32_t s = (c & 0x20u) << 26, e = (c >> 3) & 3u, m = c & 7u;
  if (e) return bitsf(s | ((e + 126u) << 23) | (m << 20));
  return bitsf(s | fbits((float)m * 0.125f));
}

MX_HD float dec_e3m2(uint32_t c) {
  uint32_t s = (c & 0x20u) << 26, e = (c >> 2) & 7u, m = c & 3u;
  if (e) return bitsf(s | ((e + 124u) << 23) | (m << 21));
  return bitsf(s | fbits((float)m * 0.0625f));
}

MX_HD float dec_e2m1(uint32_t n) {
  uint32_t s = (n & 8u) << 28, e = (n >> 1) & 3u, m = n & 1u;
  if (e) return bitsf(s | ((e + 126u) << 23) | (m << 22));
  return bitsf(s | (m ? 0x3F000000u : 0u));          // 0 or 0.5
}

// Element decoder by format (byte code for E4M3 / E5M2, 6-bit code for E2M3 / E3M2, nibble for E2M1).
MX_HD float dec_elem_fmt(int fmt, uint32_t c) {
  if (fmt == MX_E4M3) return dec_e4m3(c);
  if (fmt == MX_E5M2) return dec_e5m2(c);
  if (fmt == MX_E2M3) return dec_e2m3(c & 63u);
  if (fmt == MX_E3M2) return dec_e3m2(c & 63u);
  return dec_e2m1(c & 15u);
}

MX_HD float dec_f16(uint16_t h) {
  uint32_t s = (uint32_t)(h & 0x8000u) << 16, e = (h >> 10) & 31u, m = h & 1023u;
  if (e == 31u) return bitsf(s | 0x7F800000u | (m << 13));
  if (e) return bitsf(s | ((e + 112u) << 23) | (m << 13));
  return bitsf(s | fbits((float)m * 5.9604644775390625e-08f));  // m * 2^-24, exact
}

// fp32 -> binary16, round to nearest even, overflow to Inf, subnormals kept.
MX_HD uint16_t f32_to_f16(float f) {
  uint32_t u = fbits(f), s = (u >> 16) & 0x8000u, a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return (uint16_t)(s | 0x7E00u);
  if (a >= 0x477FF000u) return (uint16_t)(s | 0x7C00u);  // >= 65520 rounds to Inf
  if (a == 0u) return (uint16_t)s;
  int e = ilog2_bits(a);
  uint32_t sig = norm_sig(a);
  if (e >= -14) {
    uint32_t r = rne_shift(sig, 13);
    if (r == 2048u) { r = 1024u; e++; }
    return (uint16_t)(s | ((uint32_t)(e + 15) << 10) | (r - 1024u));
  }
  return (uint16_t)(s | rne_shift(sig, -1 - e));  // subnormal: multiples of 2^-24
}

}  // namespace mx
