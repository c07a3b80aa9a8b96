/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU oracle for the block-scaled quantized matmul and the
 * int8/int4 dequant matvec. Only the test suite, the smoke entry point and the CPU-baseline leg
 * of the benchmark may load this code; the product path never does. It shares no code, header,
 * table or helper with the GPU library: every decoder below is the closed form of its format,
 * every product is formed in fp64, and sums run over k in ascending order.
 *
 * Sources (the pages are cited by title and section):
 *  - "TensorOps: quantized matmul, cooperative tensors, and the neural accelerator" (Core AI model
 *    zoo notes), sections "Scale planes: one MTLTensor = data + scales" (32 data elements share
 *    one FP8 E8M0 scale), "Kernel-phase findings" (E8M0-only scale plane, block 32x1, scaled
 *    right operand stored K-contiguous; revised strategy: C += scale[b,n] * sum_{k in b} A*Wq),
 *    and "VALIDATED ON M4 MAX", fact 5 (int4 packing: C-order [K,N], two per byte, low nibble =
 *    even linear index, two's-complement nibbles).
 *  - "Optimize custom machine learning operations with Metal tensors" (WWDC26 session 330
 *    summary), sections on the auxiliary scale plane (MTLTensorDataTypeMetalFloat8UE8M0,
 *    blockFactors {32,1}: every 32 contiguous elements share one scale) and on the MXFP8
 *    matmul (E4M3 data plane, half output).
 *  - "TileLang Metal Backend Internals", section 1.4: fp32 accumulation, fp16 output by a cast
 *    at store.
 * The pages name E4M3, fp8, fp4, "MX scaling formats" and E8M0 without giving their bits (TensorOps
 * notes, quantized dtype support matrix). The readings used here are the OCP Microscaling (MX) v1.0
 * element formats: E4M3 "FN" (bias 7, S.1111.111 = NaN, no Inf, max 448), E5M2 (bias 15,
 * S.11111.00 = Inf, S.11111.xx = NaN, max 57344), the FP6 pair E2M3 (bias 1, max 7.5) and E3M2
 * (bias 3, max 28) without NaN/Inf, E2M1 (bias 1, values +-{0,.5,1,1.5,2,3,4,6}, no NaN/Inf) and
 * E8M0 (2^(e-127), 0xFF=NaN). FP6 rows are packed as a little-endian bit stream: element j in
 * bits 6j..6j+5 (4 elements in 3 bytes).
 *
 * Every function here has a pin in the CPU test suite (library dtypes, closed forms, exact
 * brute force, invariants); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_E4M3 = 0, ORC_E5M2 = 1, ORC_E2M3 = 2, ORC_E3M2 = 3, ORC_E2M1 = 4, ORC_F16 = 16, ORC_INT8 = 32, ORC_INT4 = 33 };

/* Threads the parallel loops below use from now on (test / benchmark plumbing, no arithmetic). */
void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------------------------ */
/* Decoders: closed forms of each format.                                                       */
/* ------------------------------------------------------------------------------------------ */

/* E4M3 (OCP "FN"): sign 1, exponent 4 (bias 7), mantissa 3. Exponent 0 is subnormal f*2^-9.
 * S.1111.111 is NaN; there is no infinity. */
double orc_dec_e4m3(unsigned b) {
  unsigned s = (b >> 7) & 1u, e = (b >> 3) & 15u, f = b & 7u;
  double v;
  if ((b & 0x7Fu) == 0x7Fu) return NAN;
  if (e == 0) v = ldexp((double)f, -9);
  else v = ldexp(1.0 + (double)f / 8.0, (int)e - 7);
  return s ? -v : v;
}

/* E5M2: sign 1, exponent 5 (bias 15), mantissa 2. Exponent 0 is subnormal f*2^-16. Exponent 31
 * is infinity (mantissa 0) or NaN (mantissa nonzero). */
double orc_dec_e5m2(unsigned b) {
  unsigned s = (b >> 7) & 1u, e = (b >> 2) & 31u, f = b & 3u;
  double v;
  if (e == 31) v = f ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)f, -16);
  else v = ldexp(1.0 + (double)f / 4.0, (int)e - 15);
  return s ? -v : v;
}

/* E2M3 (FP6): sign 1 (bit 5), exponent 2 (bias 1), mantissa 3. Exponent 0 is subnormal f*2^-3. */
double orc_dec_e2m3(unsigned c) {
  unsigned s = (c >> 5) & 1u, e = (c >> 3) & 3u, f = c & 7u;
  double v = e ? ldexp(1.0 + (double)f / 8.0, (int)e - 1) : ldexp((double)f, -3);
  return s ? -v : v;
}

/* E3M2 (FP6): sign 1 (bit 5), exponent 3 (bias 3), mantissa 2. Exponent 0 is subnormal f*2^-4. */
double orc_dec_e3m2(unsigned c) {
  unsigned s = (c >> 5) & 1u, e = (c >> 2) & 7u, f = c & 3u;
  double v = e ? ldexp(1.0 + (double)f / 4.0, (int)e - 3) : ldexp((double)f, -4);
  return s ? -v : v;
}

/* E2M1: sign 1, exponent 2 (bias 1), mantissa 1. Exponent 0 is subnormal 0.5*f. */
double orc_dec_e2m1(unsigned n) {
  unsigned s = (n >> 3) & 1u, e = (n >> 1) & 3u, f = n & 1u;
  double v;
  if (e == 0) v = 0.5 * (double)f;
  else v = ldexp(1.0 + (double)f / 2.0, (int)e - 1);
  return s ? -v : v;
}

/* E8M0: unsigned power of two 2^(e-127); 0xFF is NaN; 0x00 is 2^-127 (there is no zero). */
double orc_dec_e8m0(unsigned e) {
  e &= 0xFFu;
  if (e == 0xFFu) return NAN;
  return ldexp(1.0, (int)e - 127);
}

/* int4: a two's-complement nibble. */
double orc_dec_int4(unsigned n) {
  n &= 0xFu;
  return (double)((int)n - (n >= 8u ? 16 : 0));
}

/* IEEE binary16: sign 1, exponent 5 (bias 15), mantissa 10. */
double orc_dec_f16(unsigned h) {
  unsigned s = (h >> 15) & 1u, e = (h >> 10) & 31u, f = h & 1023u;
  double v;
  if (e == 31) v = f ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)f, -24);
  else v = ldexp(1.0 + (double)f / 1024.0, (int)e - 15);
  return s ? -v : v;
}

/* Element j of a row of 4-bit codes: two per byte, even index in the low nibble. */
static unsigned nibble(const uint8_t* row, int64_t j) {
  uint8_t by = row[j / 2];
  return (j % 2 == 0) ? (by & 0xFu) : (by >> 4);
}

/* Element j of a row of 6-bit codes: bits 6j..6j+5 of the row read as a little-endian bit stream. */
static unsigned sixbit(const uint8_t* row, int64_t j) {
  int64_t bit = 6 * j;
  unsigned two = (unsigned)row[bit / 8] | ((bit % 8 > 2) ? (unsigned)row[bit / 8 + 1] << 8 : 0u);
  return (two >> (bit % 8)) & 63u;
}

static int is_fp6(int fmt) { return fmt == ORC_E2M3 || fmt == ORC_E3M2; }

/* Dequantised value of element k of one MX row (codes along K, scales one per 32 along K). */
static double mx_elem(int fmt, const uint8_t* codes_row, const uint8_t* scales_row, int64_t k) {
  double v;
  if (fmt == ORC_E4M3) v = orc_dec_e4m3(codes_row[k]);
  else if (fmt == ORC_E5M2) v = orc_dec_e5m2(codes_row[k]);
  else if (fmt == ORC_E2M3) v = orc_dec_e2m3(sixbit(codes_row, k));
  else if (fmt == ORC_E3M2) v = orc_dec_e3m2(sixbit(codes_row, k));
  else v = orc_dec_e2m1(nibble(codes_row, k));
  return v * orc_dec_e8m0(scales_row[k / 32]);
}

static int64_t mx_row_bytes(int fmt, int64_t K) { return fmt == ORC_E2M1 ? K / 2 : (is_fp6(fmt) ? K / 4 * 3 : K); }

/* ------------------------------------------------------------------------------------------ */
/* MX GEMM: C[m,n] = sum_k (dec(A[m,k]) * 2^(SA[m,k/32]-127)) * (dec(B[k,n]) * 2^(SB[n,k/32]-127)) */
/* A: codes [M][K] (fp4: [M][K/2]), SA: [M][K/32]. B is K x N stored K-contiguous, i.e.          */
/* codes [N][K] (fp4: [N][K/2]) and SB: [N][K/32]. Result in fp64, k ascending.                  */
/* ------------------------------------------------------------------------------------------ */

double orc_mx_dot(int fa, int fb, int64_t K, const uint8_t* A, const uint8_t* SA, const uint8_t* B,
                  const uint8_t* SB, int64_t m, int64_t n) {
  const uint8_t* arow = A + m * mx_row_bytes(fa, K);
  const uint8_t* brow = B + n * mx_row_bytes(fb, K);
  const uint8_t* sarow = SA + m * (K / 32);
  const uint8_t* sbrow = SB + n * (K / 32);
  double acc = 0.0;
  for (int64_t k = 0; k < K; k++) acc += mx_elem(fa, arow, sarow, k) * mx_elem(fb, brow, sbrow, k);
  return acc;
}

/* Rows [row0, row0+nrows) of C, written to C[(m-row0)*N + n]. */
void orc_mxgemm_rows(int fa, int fb, int64_t M, int64_t N, int64_t K, const uint8_t* A,
                     const uint8_t* SA, const uint8_t* B, const uint8_t* SB, int64_t row0,
                     int64_t nrows, double* C) {
  (void)M;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < nrows; i++)
    for (int64_t n = 0; n < N; n++) C[i * N + n] = orc_mx_dot(fa, fb, K, A, SA, B, SB, row0 + i, n);
}

/* Selected outputs C[ms[i], ns[i]]. */
void orc_mxgemm_points(int fa, int fb, int64_t K, const uint8_t* A, const uint8_t* SA,
                       const uint8_t* B, const uint8_t* SB, const int64_t* ms, const int64_t* ns,
                       int64_t count, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; i++) out[i] = orc_mx_dot(fa, fb, K, A, SA, B, SB, ms[i], ns[i]);
}

/* ------------------------------------------------------------------------------------------ */
/* fp16 GEMM: C[m,n] = sum_k A[m,k] * B[k,n], A [M][K] and B [K][N] row-major binary16.          */
/* ------------------------------------------------------------------------------------------ */

double orc_f16_dot(int64_t N, int64_t K, const uint16_t* A, const uint16_t* B, int64_t m, int64_t n) {
  double acc = 0.0;
  for (int64_t k = 0; k < K; k++) acc += orc_dec_f16(A[m * K + k]) * orc_dec_f16(B[k * N + n]);
  return acc;
}

void orc_gemm_f16_rows(int64_t M, int64_t N, int64_t K, const uint16_t* A, const uint16_t* B,
                       int64_t row0, int64_t nrows, double* C) {
  (void)M;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < nrows; i++)
    for (int64_t n = 0; n < N; n++) C[i * N + n] = orc_f16_dot(N, K, A, B, row0 + i, n);
}

void orc_gemm_f16_points(int64_t N, int64_t K, const uint16_t* A, const uint16_t* B,
                         const int64_t* ms, const int64_t* ns, int64_t count, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; i++) out[i] = orc_f16_dot(N, K, A, B, ms[i], ns[i]);
}

/* ------------------------------------------------------------------------------------------ */
/* Dequant matvec (per 32-row block of K, one fp16 scale per column):                            */
/*   y[m,n] = sum_b Ws[b,n] * sum_{k in block b} x[m,k] * q[k,n]                                 */
/* x: binary16 [M][K]; W int8 [K][N] or int4 packed along the C-order linear index k*N+n         */
/* (two per byte, even index in the low nibble); Ws binary16 [K/32][N].                          */
/* ------------------------------------------------------------------------------------------ */

static double wq(int fw, const uint8_t* W, int64_t N, int64_t k, int64_t n) {
  if (fw == ORC_INT8) return (double)(int8_t)W[k * N + n];
  return orc_dec_int4(nibble(W, k * N + n));
}

double orc_matvec_elem(int fw, int64_t N, int64_t K, const uint16_t* x, const uint8_t* W,
                       const uint16_t* Ws, int64_t m, int64_t n) {
  double y = 0.0;
  for (int64_t b = 0; b < K / 32; b++) {
    double part = 0.0;
    for (int64_t k = 32 * b; k < 32 * b + 32; k++) part += orc_dec_f16(x[m * K + k]) * wq(fw, W, N, k, n);
    y += orc_dec_f16(Ws[b * N + n]) * part;
  }
  return y;
}

void orc_matvec(int fw, int64_t M, int64_t N, int64_t K, const uint16_t* x, const uint8_t* W,
                const uint16_t* Ws, double* y) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; n++)
    for (int64_t m = 0; m < M; m++) y[m * N + n] = orc_matvec_elem(fw, N, K, x, W, Ws, m, n);
}

/* ------------------------------------------------------------------------------------------ */
/* Dequant to fp32: out = fp32(value * scale), the exact product rounded once (C's conversion  */
/* of a double to float rounds to nearest-even and keeps subnormals).                             */
/*  MX formats: codes [rows][cols] (fp4 [rows][cols/2]), scales e8m0 [rows][cols/32].            */
/*  int8/int4:  codes [rows][cols] (int4 packed on the linear index), scales fp16 [rows/32][cols].*/
/* ------------------------------------------------------------------------------------------ */

void orc_dequant(int fmt, int64_t rows, int64_t cols, const uint8_t* codes, const void* scales, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++)
    for (int64_t c = 0; c < cols; c++) {
      double v;
      if (fmt == ORC_E4M3 || fmt == ORC_E5M2 || is_fp6(fmt) || fmt == ORC_E2M1) {
        v = mx_elem(fmt, codes + r * mx_row_bytes(fmt, cols), (const uint8_t*)scales + r * (cols / 32), c);
      } else {
        double s = orc_dec_f16(((const uint16_t*)scales)[(r / 32) * cols + c]);
        v = wq(fmt, codes, cols, r, c) * s;
      }
      out[r * cols + c] = (float)v;
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Encoders. These are encodings, so they follow the quantisation steps in order:               */
/*  1. amax of the 32-element block, 2. j = floor(log2 amax) from the exact binary exponent,     */
/*  3. E = clamp(j - emax + 127, 0, 254) with emax = 8 (E4M3), 15 (E5M2), 2 (E2M3), 4 (E3M2)   */
/*     or 2 (E2M1),                                                                            */
/*  4. v = x * 2^(127-E) exactly, 5. the element code nearest to v, ties to the even code,       */
/*     values beyond the largest finite element saturate to it, the sign is kept.              */
/* The element search is brute force over the format's own decode values (not bit arithmetic). */
/* ------------------------------------------------------------------------------------------ */

/* The positive finite element values of a format, indexed by code (E4M3: 0x00..0x7E, E5M2:
 * 0x00..0x7B, E2M1: 0..7), filled once from the closed-form decoders above. */
static double g_tab_e4m3[0x7F], g_tab_e5m2[0x7C], g_tab_e2m3[32], g_tab_e3m2[32], g_tab_e2m1[8];
static int g_tab_ready = 0;
static void build_tables(void) {
  if (g_tab_ready) return;
  for (unsigned c = 0; c < 0x7Fu; c++) g_tab_e4m3[c] = orc_dec_e4m3(c);
  for (unsigned c = 0; c < 0x7Cu; c++) g_tab_e5m2[c] = orc_dec_e5m2(c);
  for (unsigned c = 0; c < 32u; c++) g_tab_e2m3[c] = orc_dec_e2m3(c);
  for (unsigned c = 0; c < 32u; c++) g_tab_e3m2[c] = orc_dec_e3m2(c);
  for (unsigned c = 0; c < 8u; c++) g_tab_e2m1[c] = orc_dec_e2m1(c);
  g_tab_ready = 1;
}

/* Nearest finite code magnitude for |v|: brute-force search over every positive finite code,
 * ties to the even code. Values at or beyond the largest finite element saturate to it; below it
 * every candidate distance that can decide the choice is exact in fp64. */
static unsigned nearest_code(double av, int fmt) {
  const double* tab = (fmt == ORC_E4M3) ? g_tab_e4m3 : (fmt == ORC_E5M2) ? g_tab_e5m2
                      : (fmt == ORC_E2M3) ? g_tab_e2m3 : (fmt == ORC_E3M2) ? g_tab_e3m2 : g_tab_e2m1;
  unsigned best = 0, ncodes = (fmt == ORC_E4M3) ? 0x7Fu : (fmt == ORC_E5M2) ? 0x7Cu : is_fp6(fmt) ? 32u : 8u;
  double bestd = INFINITY;
  if (av >= tab[ncodes - 1u]) return ncodes - 1u;
  for (unsigned c = 0; c < ncodes; c++) {
    double d = fabs(av - tab[c]);
    if (d < bestd || (d == bestd && (c & 1u) == 0u)) { bestd = d; best = c; }
  }
  return best;
}

/* Element encoder: the code whose value is nearest to v (sign kept, -0 allowed). */
unsigned orc_enc_elem(int fmt, double v) {
  build_tables();
  unsigned mag = nearest_code(fabs(v), fmt);
  unsigned sbit = (fmt == ORC_E2M1) ? 0x8u : is_fp6(fmt) ? 0x20u : 0x80u;
  return signbit(v) ? (mag | sbit) : mag;
}

/* floor(log2 a) for finite a > 0, from the exact binary exponent: a = f * 2^e with f in [0.5,1). */
int orc_floor_log2(double a) {
  int e;
  (void)frexp(a, &e);
  return e - 1;
}

/* The E8M0 scale code of one block, from its amax (step 2-3). */
unsigned orc_mx_scale_code(int fmt, double amax) {
  int emax = (fmt == ORC_E4M3) ? 8 : (fmt == ORC_E5M2) ? 15 : (fmt == ORC_E3M2) ? 4 : 2, E;
  if (!(amax > 0.0)) return 0u; /* amax = 0: log2 is -inf, clamps to 0 */
  E = orc_floor_log2(amax) - emax + 127;
  if (E < 0) E = 0;
  if (E > 254) E = 254;
  return (unsigned)E;
}

/* Quantise rows x cols fp32 values, blocks of 32 along cols. codes [rows][cols] (fp4 packed,
 * even column in the low nibble), scales [rows][cols/32]. A block with a non-finite value gets
 * scale 0xFF and zero codes. */
void orc_mx_quantize(int fmt, int64_t rows, int64_t cols, const float* src, uint8_t* codes, uint8_t* scales) {
  int64_t rb = mx_row_bytes(fmt, cols);
  build_tables();
  memset(codes, 0, (size_t)(rows * rb));
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++)
    for (int64_t b = 0; b < cols / 32; b++) {
      const float* x = src + r * cols + 32 * b;
      double amax = 0.0;
      int finite = 1;
      for (int i = 0; i < 32; i++) {
        if (!isfinite(x[i])) finite = 0;
        else if (fabs((double)x[i]) > amax) amax = fabs((double)x[i]);
      }
      if (!finite) { scales[r * (cols / 32) + b] = 0xFFu; continue; }
      unsigned E = orc_mx_scale_code(fmt, amax);
      scales[r * (cols / 32) + b] = (uint8_t)E;
      for (int i = 0; i < 32; i++) {
        int64_t c = 32 * b + i;
        unsigned code = orc_enc_elem(fmt, ldexp((double)x[i], 127 - (int)E));
        if (fmt == ORC_E2M1) codes[r * rb + c / 2] |= (uint8_t)((c % 2 == 0) ? code : (code << 4));
        else if (is_fp6(fmt)) {
          int64_t bit = 6 * c;
          codes[r * rb + bit / 8] |= (uint8_t)(code << (bit % 8));
          if (bit % 8 > 2) codes[r * rb + bit / 8 + 1] |= (uint8_t)(code >> (8 - bit % 8));
        } else codes[r * rb + c] = (uint8_t)code;
      }
    }
}

/* Round a finite double to the nearest binary16 (ties to even) and return its bits. The value is
 * split into a quantum (the spacing of binary16 numbers around it) and rounded with rint, which
 * rounds half to even in the default rounding mode. Beyond the largest finite value (65504) the
 * result is +-Inf. */
unsigned orc_enc_f16(double x) {
  unsigned s = signbit(x) ? 0x8000u : 0u;
  double a = fabs(x), q, r;
  int j;
  if (isnan(x)) return 0x7E00u;
  if (a == 0.0) return s;
  j = orc_floor_log2(a);
  q = (j < -14) ? ldexp(1.0, -24) : ldexp(1.0, j - 10);
  r = rint(a / q) * q;
  if (r >= 65520.0 || (r > 65504.0)) return s | 0x7C00u;
  if (r < ldexp(1.0, -14)) return s | (unsigned)(r / ldexp(1.0, -24));       /* subnormal */
  j = orc_floor_log2(r);
  return s | ((unsigned)(j + 15) << 10) | (unsigned)((r / ldexp(1.0, j) - 1.0) * 1024.0);
}

/* Symmetric integer quantisation of W [K][N] (fp32), one fp16 scale per column per 32 rows:
 *   s = fp16(amax / qmax) with the division in fp32; q = clamp(rint(fp32(w / s)), -qmax, qmax),
 *   q = 0 where s = 0; a block holding Inf or NaN gets s = NaN and q = 0 (a reading: the pages
 *   never quantise non-finite weights). qmax = 127 (int8) or 7 (int4). Output q as int8 [K][N] (one per byte),
 *   scales binary16 bits [K/32][N]. Packing of int4 is separate (orc_pack_int4). */
void orc_int_quantize(int qmax, int64_t K, int64_t N, const float* w, int8_t* q, uint16_t* s16) {
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < K / 32; b++)
    for (int64_t n = 0; n < N; n++) {
      float amax = 0.0f;
      int finite = 1;
      for (int64_t k = 32 * b; k < 32 * b + 32; k++) {
        if (!isfinite(w[k * N + n])) finite = 0;
        else if (fabsf(w[k * N + n]) > amax) amax = fabsf(w[k * N + n]);
      }
      /* a block holding Inf or NaN: scale NaN (binary16 0x7E00), every q zero, so the whole block
       * dequantises to NaN (the same reading as the MX rule for non-finite blocks) */
      float ratio = amax / (float)qmax;
      unsigned sb = finite ? orc_enc_f16((double)ratio) : 0x7E00u;
      float s = (float)orc_dec_f16(sb);
      s16[b * N + n] = (uint16_t)sb;
      for (int64_t k = 32 * b; k < 32 * b + 32; k++) {
        int v = 0;
        if (finite && s != 0.0f) {
          float t = w[k * N + n] / s;
          double r = rint((double)t);
          if (r > qmax) r = qmax;
          if (r < -qmax) r = -qmax;
          v = (int)r;
        }
        q[k * N + n] = (int8_t)v;
      }
    }
}

/* int4 packing of a C-order [K][N] weight: linear index i = k*N+n, two per byte, the even index
 * in the low nibble, values as two's-complement nibbles. count = K*N (even). */
void orc_pack_int4(int64_t count, const int8_t* q, uint8_t* packed) {
  for (int64_t i = 0; i < count; i += 2)
    packed[i / 2] = (uint8_t)(((unsigned)q[i] & 0xFu) | (((unsigned)q[i + 1] & 0xFu) << 4));
}
