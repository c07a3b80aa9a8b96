// quant_rules.h -- the block quantisation rules, as plain per-block functions used by the host
// codec and by the GPU codec kernels.
//
// MX blocks (32 consecutive elements along K share one E8M0 scale: "TensorOps ... notes",
// section "Scale planes"; WWDC26 session 330 summary, auxiliary scale plane with blockFactors
// {32,1}): E = clamp(floor(log2 amax) - emax + 127, 0, 254), emax = 8 for E4M3, 15 for E5M2, 2 for
// E2M3, 4 for E3M2 and 2 for E2M1 (the exponent of the format's largest element),
// elements encoded as x * 2^(127-E). A block holding Inf/NaN gets E = 0xFF and zero codes.
//
// Integer weight blocks (32 rows of one column share one fp16 scale: the per-block fp16 scales of
// the "Kernel-phase findings" revised strategy): s = fp16(amax / qmax), q = rint(w / s) clamped to
// [-qmax, qmax], q = 0 when s = 0; a block holding Inf or NaN gets s = NaN and q = 0.
#pragma once
#include "codec_math.h"

namespace mx {

MX_HD float div_rn(float a, float b) {
#ifdef __HIP_DEVICE_COMPILE__
  return __fdiv_rn(a, b);
#else
  return a / b;
#endif
}

MX_HD float rint_even(float x) {
#ifdef __HIP_DEVICE_COMPILE__
  return __builtin_rintf(x);
#else
  return __builtin_rintf(x);  // default rounding mode: nearest, ties to even
#endif
}

constexpr int emax_of(int fmt) { return fmt == MX_E4M3 ? 8 : fmt == MX_E5M2 ? 15 : fmt == MX_E3M2 ? 4 : 2; }

// Scale code and exponent offset t = 127 - E of one MX block (element format fmt) from its amax
// bit pattern and a non-finite flag. Returns the scale code; *t receives the offset.
MX_HD uint32_t mx_block_scale(uint32_t amax_bits, bool nonfinite, int fmt, int* t) {
  if (nonfinite) { *t = 0; return 0xFFu; }
  uint32_t E = scale_code(amax_bits, emax_of(fmt));
  *t = 127 - (int)E;
  return E;
}

// Integer symmetric quantisation of one weight given the block's fp16 scale (as fp32). A zero
// scale (all-zero block) and a NaN scale (block holding Inf or NaN) give 0, so the cast below only
// ever sees a finite value.
MX_HD int int_quant(float w, float s, int qmax) {
  if (!(s > 0.0f)) return 0;
  float r = rint_even(div_rn(w, s));
  r = r > (float)qmax ? (float)qmax : r;
  r = r < (float)-qmax ? (float)-qmax : r;
  return (int)r;
}

// fp16 block scale (bits) of an integer weight block from its amax; a block holding Inf or NaN
// gets the NaN scale 0x7E00 (its codes are all 0, so it dequantises to NaN, as an MX block does).
MX_HD uint16_t int_block_scale(float amax, bool nonfinite, int qmax) {
  return nonfinite ? (uint16_t)0x7E00u : f32_to_f16(div_rn(amax, (float)qmax));
}

}  // namespace mx
