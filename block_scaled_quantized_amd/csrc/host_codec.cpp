// host_codec.cpp -- host (CPU) pack/unpack of the MX and integer weight formats.
// Same rules and layouts as the GPU codec kernels (codec.hip); see mxgemm.h for the contract.
#include <cmath>
#include <cstring>

#include "quant_rules.h"

using namespace mx;

namespace {

bool is_mx(int f) { return f == MX_E4M3 || f == MX_E5M2 || f == MX_E2M3 || f == MX_E3M2 || f == MX_E2M1; }

// Row bytes of an MX row of n elements.
int64_t mx_row_bytes(int f, int64_t n) { return is_byte_fmt(f) ? n : (is_fp6_fmt(f) ? n / 4 * 3 : n / 2); }
bool is_int(int f) { return f == MX_INT8 || f == MX_INT4; }

int pack_mx(int fmt, const float* src, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales) {
  const bool byte = is_byte_fmt(fmt), fp6 = is_fp6_fmt(fmt);
  const int64_t rb = mx_row_bytes(fmt, cols), nb = cols / 32, bb = byte ? 32 : (fp6 ? 24 : 16);
  for (int64_t r = 0; r < rows; r++)
    for (int64_t b = 0; b < nb; b++) {
      const float* x = src + r * cols + 32 * b;
      uint32_t amax = 0u;
      bool nonfinite = false;
      for (int i = 0; i < 32; i++) {
        uint32_t a = fbits(x[i]) & 0x7FFFFFFFu;
        nonfinite |= a >= 0x7F800000u;
        amax = a > amax ? a : amax;  // magnitude order equals bit order for finite floats
      }
      int t;
      scales[r * nb + b] = (uint8_t)mx_block_scale(amax, nonfinite, fmt, &t);
      uint8_t* out = codes + r * rb + bb * b;
      if (nonfinite) { memset(out, 0, (size_t)bb); continue; }
      if (byte) {
        for (int i = 0; i < 32; i++) out[i] = (uint8_t)enc_elem_fmt(fmt, x[i], t);
      } else if (fp6) {  // 4 elements per 3 bytes, little-endian bit stream
        for (int q = 0; q < 8; q++) {
          uint32_t w = 0u;
          for (int i = 0; i < 4; i++) w |= enc_elem_fmt(fmt, x[4 * q + i], t) << (6 * i);
          out[3 * q] = (uint8_t)w;
          out[3 * q + 1] = (uint8_t)(w >> 8);
          out[3 * q + 2] = (uint8_t)(w >> 16);
        }
      } else {
        for (int i = 0; i < 16; i++)
          out[i] = (uint8_t)(enc_elem_fmt(fmt, x[2 * i], t) | (enc_elem_fmt(fmt, x[2 * i + 1], t) << 4));
      }
    }
  return MX_OK;
}

int pack_int(bool i8, const float* w, int64_t K, int64_t N, uint8_t* codes, uint16_t* scales) {
  const int qmax = i8 ? 127 : 7;
  if (!i8) memset(codes, 0, (size_t)(K * N / 2));
  for (int64_t b = 0; b < K / 32; b++)
    for (int64_t n = 0; n < N; n++) {
      float amax = 0.0f;
      bool nonfinite = false;
      for (int64_t k = 32 * b; k < 32 * b + 32; k++) {
        amax = std::fmax(amax, std::fabs(w[k * N + n]));
        nonfinite |= !std::isfinite(w[k * N + n]);
      }
      uint16_t sb = int_block_scale(amax, nonfinite, qmax);
      scales[b * N + n] = sb;
      float s = dec_f16(sb);
      for (int64_t k = 32 * b; k < 32 * b + 32; k++) {
        int q = int_quant(w[k * N + n], s, qmax);
        if (i8) {
          codes[k * N + n] = (uint8_t)(int8_t)q;
        } else {
          int64_t i = k * N + n;
          codes[i / 2] |= (uint8_t)(((unsigned)q & 0xFu) << (4 * (i % 2)));
        }
      }
    }
  return MX_OK;
}

}  // namespace

extern "C" int mx_pack_host(int f, const float* src, int64_t rows, int64_t cols, void* codes, void* scales) {
  if (!src || !codes || !scales) return MX_ERR_NULL;
  if (rows < 1 || cols < 1 || rows > MX_MAX_DIM || cols > MX_MAX_DIM) return MX_ERR_SHAPE;
  if (is_mx(f)) {
    if (cols % 32) return MX_ERR_SHAPE;
    return pack_mx(f, src, rows, cols, (uint8_t*)codes, (uint8_t*)scales);
  }
  if (is_int(f)) {
    if (rows % 32 || (f == MX_INT4 && cols % 2)) return MX_ERR_SHAPE;
    return pack_int(f == MX_INT8, src, rows, cols, (uint8_t*)codes, (uint16_t*)scales);
  }
  return MX_ERR_FORMAT;
}

extern "C" int mx_unpack_host(int f, const void* codes_v, const void* scales_v, int64_t rows, int64_t cols, float* out) {
  if (!codes_v || !scales_v || !out) return MX_ERR_NULL;
  if (rows < 1 || cols < 1 || rows > MX_MAX_DIM || cols > MX_MAX_DIM) return MX_ERR_SHAPE;
  const uint8_t* codes = (const uint8_t*)codes_v;
  if (is_mx(f)) {
    if (cols % 32) return MX_ERR_SHAPE;
    const uint8_t* sc = (const uint8_t*)scales_v;
    const bool byte = is_byte_fmt(f), fp6 = is_fp6_fmt(f);
    const int64_t rb = mx_row_bytes(f, cols);
    for (int64_t r = 0; r < rows; r++)
      for (int64_t c = 0; c < cols; c++) {
        uint32_t code;
        if (byte) code = codes[r * rb + c];
        else if (fp6) {
          const uint8_t* g = codes + r * rb + 3 * (c / 4);  // the 3 bytes of c's group of 4
          code = (((uint32_t)g[0] | ((uint32_t)g[1] << 8) | ((uint32_t)g[2] << 16)) >> (6 * (c % 4))) & 63u;
        } else code = (codes[r * rb + c / 2] >> (4 * (c % 2))) & 0xFu;
        float v = dec_elem_fmt(f, code);
        out[r * cols + c] = v * dec_e8m0(sc[r * (cols / 32) + c / 32]);
      }
    return MX_OK;
  }
  if (is_int(f)) {
    if (rows % 32 || (f == MX_INT4 && cols % 2)) return MX_ERR_SHAPE;
    const uint16_t* sc = (const uint16_t*)scales_v;
    for (int64_t r = 0; r < rows; r++)
      for (int64_t c = 0; c < cols; c++) {
        int64_t i = r * cols + c;
        int q = f == MX_INT8 ? (int)(int8_t)codes[i] : (((int)((codes[i / 2] >> (4 * (i % 2))) & 0xFu) ^ 8) - 8);
        out[i] = (float)q * dec_f16(sc[(r / 32) * cols + c]);
      }
    return MX_OK;
  }
  return MX_ERR_FORMAT;
}

extern "C" uint8_t mx_encode_host(int f, float v) {
  if (is_mx(f)) return (uint8_t)enc_elem_fmt(f, v, 0);
  return 0;
}

extern "C" float mx_decode_host(int f, uint8_t code) {
  switch (f) {
    case MX_E4M3: return dec_e4m3(code);
    case MX_E5M2: return dec_e5m2(code);
    case MX_E2M3: return dec_e2m3(code & 63u);
    case MX_E3M2: return dec_e3m2(code & 63u);
    case MX_E2M1: return dec_e2m1(code & 0xFu);
    case MX_INT8: return (float)(int8_t)code;
    case MX_INT4: return (float)((int)((code & 0xFu) ^ 8u) - 8);
    case MX_E8M0: return dec_e8m0(code);
    default: return bitsf(0x7FC00000u);
  }
}
