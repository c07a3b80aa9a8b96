// codec.hip -- GPU pack (quantise) and unpack (dequantise) kernels for the MX and integer
// weight formats. Same rules as the host codec (quant_rules.h), hence bit-identical results.
//
// MX pack: 8 lanes own one 32-element block (4 elements each, one 16-byte load per lane); the
// block amax and the non-finite flag are reduced over those 8 lanes with xor shuffles; every lane
// then encodes its 4 elements into one 32-bit (E4M3, E5M2) or 16-bit (E2M1) store. A wave covers eight
// consecutive blocks, i.e. 1 KiB of contiguous fp32 input. E4M3 and E2M1 encode with gfx950's
// scaled conversions, which give the rule's codes exactly (see pack_mx_kernel); E5M2 and the FP6
// formats with the rule's integer arithmetic.
#include "quant_rules.h"

using namespace mx;

namespace {

constexpr int kThreads = 256;
typedef short v2s16 __attribute__((ext_vector_type(2)));

template <int FMT>
__global__ __launch_bounds__(kThreads) void pack_mx_kernel(const float* __restrict__ src,
                                                           int64_t nblocks,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
  const int sub = threadIdx.x & 7;
  const int64_t stride = (int64_t)gridDim.x * (kThreads / 8);
  for (int64_t blk = (int64_t)blockIdx.x * (kThreads / 8) + (threadIdx.x >> 3); blk < nblocks; blk += stride) {
    const float4 v = reinterpret_cast<const float4*>(src)[blk * 8 + sub];
    const float x[4] = {v.x, v.y, v.z, v.w};
    uint32_t amax = 0u, nonfinite = 0u;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      uint32_t a = fbits(x[i]) & 0x7FFFFFFFu;
      nonfinite |= (uint32_t)(a >= 0x7F800000u);
      amax = a > amax ? a : amax;
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
      uint32_t o = (uint32_t)__shfl_xor((int)amax, off, 8);
      amax = o > amax ? o : amax;
      nonfinite |= (uint32_t)__shfl_xor((int)nonfinite, off, 8);
    }
    int t;
    const uint32_t E = mx_block_scale(amax, nonfinite != 0u, FMT, &t);
    if (sub == 0) scales[blk] = (uint8_t)E;  // scales [rows][cols/32]: block blk's byte is byte blk
    if constexpr (FMT == MX_E4M3) {
      // gfx950's scaled conversion divides by 2^(E-127) (the scale passed as the bit pattern E << 23,
      // which it reads as an exponent, E = 0 included) and rounds to nearest even, as the rule
      // does; it writes NaN (S.1111.111) where the scaled value exceeds 464 instead of saturating,
      // and those bytes become S.1111.110 (+-448). Checked on the box against the encoder below
      // for every mantissa of every fp32 exponent that scales to 2^-40..2^8, both signs, at scale
      // codes from 0 to 254 (fp32 subnormal inputs included): no difference.
      const float scale = __builtin_bit_cast(float, E << 23);
      v2s16 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((v2s16){0, 0}, x[0], x[1], scale, false);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, x[2], x[3], scale, true);
      uint32_t w = __builtin_bit_cast(uint32_t, r);
      const uint32_t m = w & 0x7F7F7F7Fu, nan = (m + 0x01010101u) & 0x80808080u;  // bytes S.1111.111
      w ^= nan >> 7;                                                              // -> S.1111.110
      reinterpret_cast<uint32_t*>(codes)[blk * 8 + sub] = nonfinite ? 0u : w;
    } else if constexpr (is_byte_fmt(FMT)) {
      uint32_t w = 0u;
      if (!nonfinite) {
#pragma unroll
        for (int i = 0; i < 4; i++) w |= enc_elem_fmt(FMT, x[i], t) << (8 * i);
      }
      reinterpret_cast<uint32_t*>(codes)[blk * 8 + sub] = w;
    } else if constexpr (is_fp6_fmt(FMT)) {  // 24 bits per lane: bytes 3 sub.. of the block's 24
      uint32_t w = 0u;
      if (!nonfinite) {
#pragma unroll
        for (int i = 0; i < 4; i++) w |= enc_elem_fmt(FMT, x[i], t) << (6 * i);
      }
      uint8_t* o = codes + blk * 24 + 3 * sub;
      o[0] = (uint8_t)w;
      o[1] = (uint8_t)(w >> 8);
      o[2] = (uint8_t)(w >> 16);
    } else {
      // E2M1 by the scaled conversion as for E4M3 (it saturates to +-6 itself; the same check,
      // over scaled exponents -40..2, found no difference), two elements per byte, the first in
      // the low nibble
      const float scale = __builtin_bit_cast(float, E << 23);
      uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[0], x[1], scale, 0);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2], x[3], scale, 1);
      reinterpret_cast<uint16_t*>(codes)[blk * 8 + sub] = nonfinite ? (uint16_t)0u : (uint16_t)w;
    }
  }
}

// Integer weights: one thread per (32-row block, column pair); columns are contiguous across
// threads, so every row access of a wave is coalesced.
__global__ __launch_bounds__(kThreads) void pack_int_kernel(bool i8, const float* __restrict__ w, int K, int N,
                                                            uint8_t* __restrict__ codes,
                                                            uint16_t* __restrict__ scales) {
  const int pairs = (N + 1) / 2;
  const int64_t total = (int64_t)(K / 32) * pairs;
  const int qmax = i8 ? 127 : 7;
  for (int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x; id < total; id += (int64_t)gridDim.x * kThreads) {
    const int b = (int)(id / pairs), n0 = 2 * (int)(id % pairs);
    const bool two = n0 + 1 < N;
    float amax0 = 0.0f, amax1 = 0.0f;
    bool nf0 = false, nf1 = false;
    for (int k = 32 * b; k < 32 * b + 32; k++) {
      const float w0 = w[(int64_t)k * N + n0];
      amax0 = fmaxf(amax0, fabsf(w0));
      nf0 |= !__builtin_isfinite(w0);
      if (two) {
        const float w1 = w[(int64_t)k * N + n0 + 1];
        amax1 = fmaxf(amax1, fabsf(w1));
        nf1 |= !__builtin_isfinite(w1);
      }
    }
    const uint16_t sb0 = int_block_scale(amax0, nf0, qmax), sb1 = int_block_scale(amax1, nf1, qmax);
    scales[(int64_t)b * N + n0] = sb0;
    if (two) scales[(int64_t)b * N + n0 + 1] = sb1;
    const float s0 = dec_f16(sb0), s1 = dec_f16(sb1);
    for (int k = 32 * b; k < 32 * b + 32; k++) {
      const int64_t i = (int64_t)k * N + n0;
      const int q0 = int_quant(w[i], s0, qmax);
      const int q1 = two ? int_quant(w[i + 1], s1, qmax) : 0;
      if (i8) {
        codes[i] = (uint8_t)(int8_t)q0;
        if (two) codes[i + 1] = (uint8_t)(int8_t)q1;
      } else {
        codes[i / 2] = (uint8_t)(((unsigned)q0 & 0xFu) | (((unsigned)q1 & 0xFu) << 4));  // N even
      }
    }
  }
}

// MX unpack: one thread per 4 consecutive elements of a row (cols % 32 == 0).
template <int FMT>
__global__ __launch_bounds__(kThreads) void unpack_mx_kernel(const uint8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ scales, int64_t nquads,
                                                             float* __restrict__ out) {
  for (int64_t qd = (int64_t)blockIdx.x * kThreads + threadIdx.x; qd < nquads; qd += (int64_t)gridDim.x * kThreads) {
    // scales [rows][cols/32] with cols % 32 == 0: element e's scale is byte e / 32, so quad qd's is
    // byte qd / 8 (no division by the row length)
    const float s = dec_e8m0(scales[qd >> 3]);
    uint32_t w;
    if constexpr (is_byte_fmt(FMT)) w = reinterpret_cast<const uint32_t*>(codes)[qd];
    else if constexpr (is_fp6_fmt(FMT))
      w = (uint32_t)codes[3 * qd] | ((uint32_t)codes[3 * qd + 1] << 8) | ((uint32_t)codes[3 * qd + 2] << 16);
    else w = reinterpret_cast<const uint16_t*>(codes)[qd];
    float4 o;
    if constexpr (is_fp6_fmt(FMT)) {
      o = make_float4(dec_elem_fmt(FMT, w & 63u) * s, dec_elem_fmt(FMT, (w >> 6) & 63u) * s,
                      dec_elem_fmt(FMT, (w >> 12) & 63u) * s, dec_elem_fmt(FMT, (w >> 18) & 63u) * s);
    } else if constexpr (is_byte_fmt(FMT)) {
      o = make_float4(dec_elem_fmt(FMT, w & 255u) * s, dec_elem_fmt(FMT, (w >> 8) & 255u) * s,
                      dec_elem_fmt(FMT, (w >> 16) & 255u) * s, dec_elem_fmt(FMT, w >> 24) * s);
    } else {
      o = make_float4(dec_e2m1(w & 15u) * s, dec_e2m1((w >> 4) & 15u) * s, dec_e2m1((w >> 8) & 15u) * s,
                      dec_e2m1((w >> 12) & 15u) * s);
    }
    reinterpret_cast<float4*>(out)[qd] = o;
  }
}

// Integer unpack: one thread per element; the fp16 scale is shared by 32 rows of a column.
__global__ __launch_bounds__(kThreads) void unpack_int_kernel(bool i8, const uint8_t* __restrict__ codes,
                                                              const uint16_t* __restrict__ scales, int64_t total,
                                                              int64_t cols, float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kThreads) {
    const int64_t r = i / cols, c = i % cols;
    int q;
    if (i8) q = (int)(int8_t)codes[i];
    else q = (int)(((codes[i / 2] >> (4 * (i & 1))) & 0xFu) ^ 8u) - 8;
    out[i] = (float)q * dec_f16(scales[(r / 32) * cols + c]);
  }
}

int grid_for(int64_t work_items, int per_block) {
  int64_t g = (work_items + per_block - 1) / per_block;
  return (int)(g < 1 ? 1 : (g > 65536 ? 65536 : g));
}

}  // namespace

extern "C" int mx_pack_run(int f, const float* src, int rows, int cols, void* codes, void* scales, void* stream) {
  if (!src || !codes || !scales) return MX_ERR_NULL;
  if (rows < 1 || cols < 1 || rows > MX_MAX_DIM || cols > MX_MAX_DIM) return MX_ERR_SHAPE;
  if (!aligned16(src) || !aligned16(codes) || !aligned16(scales)) return MX_ERR_ALIGN;
  hipStream_t st = as_stream(stream);
  if (f == MX_E4M3 || f == MX_E5M2 || f == MX_E2M3 || f == MX_E3M2 || f == MX_E2M1) {
    if (cols % 32) return MX_ERR_SHAPE;
    if (int a = check_arch()) return a;
    const int64_t nblocks = (int64_t)rows * (cols / 32);
    const dim3 grid(grid_for(nblocks, kThreads / 8)), block(kThreads);
    if (f == MX_E4M3)
      hipLaunchKernelGGL(pack_mx_kernel<MX_E4M3>, grid, block, 0, st, src, nblocks, (uint8_t*)codes, (uint8_t*)scales);
    else if (f == MX_E5M2)
      hipLaunchKernelGGL(pack_mx_kernel<MX_E5M2>, grid, block, 0, st, src, nblocks, (uint8_t*)codes, (uint8_t*)scales);
    else if (f == MX_E2M3)
      hipLaunchKernelGGL(pack_mx_kernel<MX_E2M3>, grid, block, 0, st, src, nblocks, (uint8_t*)codes, (uint8_t*)scales);
    else if (f == MX_E3M2)
      hipLaunchKernelGGL(pack_mx_kernel<MX_E3M2>, grid, block, 0, st, src, nblocks, (uint8_t*)codes, (uint8_t*)scales);
    else
      hipLaunchKernelGGL(pack_mx_kernel<MX_E2M1>, grid, block, 0, st, src, nblocks, (uint8_t*)codes, (uint8_t*)scales);
    return sync_check(launch_status(), st);
  }
  if (f == MX_INT8 || f == MX_INT4) {
    if (rows % 32 || (f == MX_INT4 && cols % 2)) return MX_ERR_SHAPE;
    if (int a = check_arch()) return a;
    const int64_t items = (int64_t)(rows / 32) * ((cols + 1) / 2);
    hipLaunchKernelGGL(pack_int_kernel, dim3(grid_for(items, kThreads)), dim3(kThreads), 0, st, f == MX_INT8, src,
                       rows, cols, (uint8_t*)codes, (uint16_t*)scales);
    return sync_check(launch_status(), st);
  }
  return MX_ERR_FORMAT;
}

extern "C" int mx_unpack_run(int f, const void* codes, const void* scales, int rows, int cols, float* out,
                             void* stream) {
  if (!codes || !scales || !out) return MX_ERR_NULL;
  if (rows < 1 || cols < 1 || rows > MX_MAX_DIM || cols > MX_MAX_DIM) return MX_ERR_SHAPE;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(out)) return MX_ERR_ALIGN;
  hipStream_t st = as_stream(stream);
  if (f == MX_E4M3 || f == MX_E5M2 || f == MX_E2M3 || f == MX_E3M2 || f == MX_E2M1) {
    if (cols % 32) return MX_ERR_SHAPE;
    if (int a = check_arch()) return a;
    const int64_t nquads = (int64_t)rows * cols / 4;
    const dim3 grid(grid_for(nquads, kThreads)), block(kThreads);
    const uint8_t *cd = (const uint8_t*)codes, *sc = (const uint8_t*)scales;
    if (f == MX_E4M3)
      hipLaunchKernelGGL(unpack_mx_kernel<MX_E4M3>, grid, block, 0, st, cd, sc, nquads, out);
    else if (f == MX_E5M2)
      hipLaunchKernelGGL(unpack_mx_kernel<MX_E5M2>, grid, block, 0, st, cd, sc, nquads, out);
    else if (f == MX_E2M3)
      hipLaunchKernelGGL(unpack_mx_kernel<MX_E2M3>, grid, block, 0, st, cd, sc, nquads, out);
    else if (f == MX_E3M2)
      hipLaunchKernelGGL(unpack_mx_kernel<MX_E3M2>, grid, block, 0, st, cd, sc, nquads, out);
    else
      hipLaunchKernelGGL(unpack_mx_kernel<MX_E2M1>, grid, block, 0, st, cd, sc, nquads, out);
    return sync_check(launch_status(), st);
  }
  if (f == MX_INT8 || f == MX_INT4) {
    if (rows % 32 || (f == MX_INT4 && cols % 2)) return MX_ERR_SHAPE;
    if (int a = check_arch()) return a;
    const int64_t total = (int64_t)rows * cols;
    hipLaunchKernelGGL(unpack_int_kernel, dim3(grid_for(total, kThreads)), dim3(kThreads), 0, st, f == MX_INT8,
                       (const uint8_t*)codes, (const uint16_t*)scales, total, (int64_t)cols, out);
    return sync_check(launch_status(), st);
  }
  return MX_ERR_FORMAT;
}
