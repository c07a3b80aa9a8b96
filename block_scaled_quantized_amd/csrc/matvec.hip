// matvec.hip -- int8 / int4 dequant matvec for decode (M <= 8 activation rows), and the same
// product at 9 <= M <= 256 rows (gemm_wq_kernel below).
//
//   y[m,n] = sum_b Ws[b,n] * sum_{k in block b} x[m,k] * q[k,n]     (32-row blocks b)
//
// the per-block fp16-scale form of "TensorOps ... notes", section "Kernel-phase findings"
// (revised strategy), with the int4 packing of section "VALIDATED ON M4 MAX", fact 5.
//
// The weight matrix is the only large operand, so the kernel is organised around streaming it
// exactly once from HBM with many bytes in flight per CU:
//  - A workgroup owns a strip of TW = 16*C columns over the whole of K, so every output is
//    finished by one workgroup (no partial sums leave the chip, no second pass, no scratch).
//  - Its W waves split K: wave w takes the 32-row blocks w, w+W, w+2W, ...
//  - One 32-row block of the strip is one fp16 MFMA 16x16x32 per column offset j < C:
//      A (16 x 32) = x rows 0..15 of the block (rows >= M repeat row M-1; their results are dropped),
//      B (32 x 16) = exact fp16 weights of the columns col0 + C*i + j, i = 0..15,
//    so lane l (i = l%16, q = l/16) loads rows 8q..8q+7 of the block for its C adjacent columns
//    and needs no cross-lane exchange. The MFMA does the M-fold reuse of every weight, which
//    keeps the vector ALU work per weight independent of M.
//  - Weights become exact fp16 pairs (q[k,n], q[k+1,n]) by the usual magic-number conversion
//    (a small integer placed in the significand of fp16 1024 reads as 1024 + integer, so one
//    subtraction of the bias recovers it exactly): one byte permute, one xor that plants the fp16
//    exponent of 1024 and the offset-binary bit, and one packed fp16 subtract.
//  - The block's fp32 product is multiplied by the fp16 block scale of its column and added to
//    an fp32 accumulator; the waves' accumulators meet in LDS, and the sum is rounded once to
//    fp16.
//  - Loads run P blocks ahead of the MFMAs through a ring of registers.
#include <mutex>

#include "codec_math.h"

using namespace mx;

namespace {

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

MX_DEV v2h as_v2h(uint32_t u) { return __builtin_bit_cast(v2h, u); }

// One block's loads for one lane: 8 weight rows (C columns each), the lane's x fragment of each of
// MT 16-row activation tiles and the C block scales.
template <bool I8, int C, int MT = 1>
struct Stage {
  static constexpr int kWordsPerRow = I8 ? C / 4 : C / 8 > 0 ? C / 8 : 1;
  uint32_t w[8][kWordsPerRow];
  uint4 xa[MT];
  uint32_t sc[C / 2];
};

// Buffer resource over `bytes` bytes at `base` (raw buffer, no swizzle); lane offsets stay 32-bit.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
MX_DEV rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Per-lane, loop-invariant byte offsets of the loads (lanes past N or M read in-range data whose
// products land only in dropped outputs).
struct LaneOffsets {
  uint32_t w;   // weight row 8q of a block, the lane's first column
  uint32_t x;   // activation row, element 8q of a block
  uint32_t s;   // block scale of the lane's first column
  uint32_t xt;  // bytes between the activation tiles (16 rows)
};

// Loads of block `blk`: W rows 32*blk + 8q + r (r < 8) of the lane's C columns, its C block scales
// and (XG) its x fragment. The weight and scale resources are rebased per block, so offsets stay small
// for any matrix size.
template <bool I8, int C, bool XG, int MT = 1, int WPOL = 0>
MX_DEV void load_stage(Stage<I8, C, MT>& s, const uint8_t* __restrict__ Wt, rsrc_t xr, const _Float16* __restrict__ Ws,
                       uint32_t N, int blk, const LaneOffsets& lo) {
  const uint32_t row_bytes = I8 ? N : N / 2;
  const rsrc_t wr = make_rsrc(Wt + (int64_t)blk * 32 * row_bytes, 32u * row_bytes);
  constexpr int WPR = Stage<I8, C, MT>::kWordsPerRow;
#pragma unroll
  for (int r = 0; r < 8; r++) {
    const int so = (int)(r * row_bytes);
    if constexpr (!I8 && C == 4) {
      s.w[r][0] = __builtin_amdgcn_raw_buffer_load_b16(wr, (int)lo.w, so, WPOL);
    } else if constexpr (WPR == 1) {
      s.w[r][0] = __builtin_amdgcn_raw_buffer_load_b32(wr, (int)lo.w, so, WPOL);
    } else if constexpr (WPR == 2) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(wr, (int)lo.w, so, WPOL);
      s.w[r][0] = v[0];
      s.w[r][1] = v[1];
    } else {
      static_assert(WPR == 4, "4, 8, 16 int8 or 4, 8, 16, 32 int4 columns per lane");
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(wr, (int)lo.w, so, WPOL);
#pragma unroll
      for (int e = 0; e < 4; e++) s.w[r][e] = v[e];
    }
  }
  if constexpr (XG) {
#pragma unroll
    for (int t = 0; t < MT; t++) {
      const auto xv = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)(lo.x + t * lo.xt), blk * 64, 0);
      s.xa[t] = make_uint4(xv[0], xv[1], xv[2], xv[3]);
    }
  }
  const rsrc_t sr = make_rsrc(Ws + (int64_t)blk * N, 2u * N);
  if constexpr (C == 4) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(sr, (int)lo.s, 0, WPOL);
    s.sc[0] = v[0];
    s.sc[1] = v[1];
  } else {
#pragma unroll
    for (int h = 0; h < C / 8; h++) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(sr, (int)lo.s + 16 * h, 0, WPOL);
#pragma unroll
      for (int e = 0; e < 4; e++) s.sc[4 * h + e] = v[e];
    }
  }
}

// fp16 pair (lo = byte a of word u0, hi = byte b of word u1) as an exact fp16 pair of the
// integers, given offset-binary conversion: bytes xor `flip` give 1024 + q + bias, minus `bias2`.
MX_DEV uint32_t pick_pair(uint32_t u1, uint32_t u0, uint32_t sel) { return __builtin_amdgcn_perm(u1, u0, sel); }

// B fragments of one block for the 4 columns 4g..4g+3 of the lane: frag[e] = the 8 fp16 weights
// (rows 8q..8q+7) of column 4g+e, as pairs (q[2p][c], q[2p+1][c]).
template <bool I8, int C, int MT>
MX_DEV void weights_to_frags(const Stage<I8, C, MT>& s, int g, v8h (&frag)[4]) {
  uint32_t f[4][4];
  if constexpr (I8) {
    // fp16 bits 0x64XX = 1024 + XX; XX = q ^ 0x80 = q + 128, so subtract 1152 (0x6480).
    const v2h bias = as_v2h(0x64806480u);
#pragma unroll
    for (int p = 0; p < 4; p++)
#pragma unroll
      for (int b = 0; b < 4; b++) {
        // byte b of word g of row 2p (low half) and of row 2p+1 (high half), zero elsewhere
        const uint32_t sel = (uint32_t)b | (0x0Cu << 8) | ((uint32_t)(4 + b) << 16) | (0x0Cu << 24);
        const uint32_t pr = pick_pair(s.w[2 * p + 1][g], s.w[2 * p][g], sel) ^ 0x64806480u;
        f[b][p] = __builtin_bit_cast(uint32_t, as_v2h(pr) - bias);
      }
  } else {
    // nibble u (two's complement q) ^ 8 = q + 8; fp16 1024 + q + 8, subtract 1032 (0x6408).
    const v2h bias = as_v2h(0x64086408u);
#pragma unroll
    for (int p = 0; p < 4; p++) {
      if constexpr (C == 4) {
        // rows 2p, 2p+1: 4 nibbles each (columns 0..3, even column in the low nibble)
        const uint32_t d = s.w[2 * p][0] | (s.w[2 * p + 1][0] << 16);
        const uint32_t e = d & 0x0F0F0F0Fu, o = (d >> 4) & 0x0F0F0F0Fu;  // cols 0,2 | 1,3 (row 2p: bytes 0,1)
        f[0][p] = __builtin_bit_cast(uint32_t, as_v2h(pick_pair(e, e, 0x0C020C00u) ^ 0x64086408u) - bias);
        f[1][p] = __builtin_bit_cast(uint32_t, as_v2h(pick_pair(o, o, 0x0C020C00u) ^ 0x64086408u) - bias);
        f[2][p] = __builtin_bit_cast(uint32_t, as_v2h(pick_pair(e, e, 0x0C030C01u) ^ 0x64086408u) - bias);
        f[3][p] = __builtin_bit_cast(uint32_t, as_v2h(pick_pair(o, o, 0x0C030C01u) ^ 0x64086408u) - bias);
      } else {
        // word g/2 of rows 2p, 2p+1 holds 8 nibbles (column 2b in the low nibble of byte b); this
        // group is its bytes 2*(g%2) and 2*(g%2)+1. With every nibble xor 8 (offset binary q + 8),
        // byte b of both rows goes to bits 0-7 and 16-23; the low nibbles or'ed into fp16 1024
        // give 1024 + q + 8 (subtract 1032), the high nibbles give 1024 + 16 (q + 8) (times 1/16,
        // minus 72): one permute, two and-or and one packed fp16 op per pair of weights, all exact.
        // (the masks and the exponent live in VGPRs, so each and-or is one v_and_or_b32: a VOP3
        // instruction cannot take two literal constants)
        uint32_t m_lo, m_hi, e_one;
        asm("v_mov_b32 %0, 0x000f000f" : "=v"(m_lo));
        asm("v_mov_b32 %0, 0x00f000f0" : "=v"(m_hi));
        asm("v_mov_b32 %0, 0x64006400" : "=v"(e_one));
        const uint32_t ua = s.w[2 * p][g / 2] ^ 0x88888888u, ub = s.w[2 * p + 1][g / 2] ^ 0x88888888u;
#pragma unroll
        for (int h = 0; h < 2; h++) {
          const uint32_t b = 2u * (uint32_t)(g % 2) + (uint32_t)h;
          const uint32_t sel = b | (0x0Cu << 8) | ((4u + b) << 16) | (0x0Cu << 24);
          const uint32_t xb = pick_pair(ub, ua, sel);
          const v2h lo = as_v2h((xb & m_lo) | e_one), hi = as_v2h((xb & m_hi) | e_one);
          f[2 * h][p] = __builtin_bit_cast(uint32_t, lo - bias);
          f[2 * h + 1][p] = __builtin_bit_cast(uint32_t, hi * as_v2h(0x2C002C00u) - as_v2h(0x54805480u));
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 4; e++) frag[e] = __builtin_bit_cast(v8h, make_uint4(f[e][0], f[e][1], f[e][2], f[e][3]));
}

// One block: per group of 4 columns, the 4 block products (MFMA, fp32) scaled by their columns'
// fp16 block scales and added to the accumulators. VM: output rows 4q + v, v < VM, that are scaled
// (VM = 1 when only activation row 0 exists: the other rows of the product are never stored).
template <bool I8, int C, int VM = 4>
MX_DEV void compute_stage(const Stage<I8, C>& s, const v8h xa, v4f (&acc)[C]) {
#pragma unroll
  for (int g = 0; g < C / 4; g++) {
    v8h frag[4];
    weights_to_frags<I8, C>(s, g, frag);
    v4f d[4];  // independent products first, so the MFMAs pipeline
#pragma unroll
    for (int e = 0; e < 4; e++) d[e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, frag[e], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const int j = 4 * g + e;
      const v2h sp = as_v2h(s.sc[j / 2]);
      const float sj = (float)sp[j & 1];
#pragma unroll
      for (int v = 0; v < VM; v++) acc[j][v] = __builtin_fmaf(sj, d[e][v], acc[j][v]);
    }
  }
}

// Single-pass kernel (no workspace): one workgroup owns a column strip of TW = 16*C columns over
// all of K. Its W waves take every W-th 32-row block, each wave covering all TW columns, so with 8
// int8 columns per lane a load instruction reads whole 128-byte lines of 4 rows (int4: 64-byte
// halves, for twice the workgroups). The waves' sums meet in LDS and the workgroup writes y.
constexpr int kXsMax = 16384;  // activation halfs staged in LDS per workgroup (M * K)
// Cache policy of the single-pass weight and scale loads: sc0 nt (past the L1, non-temporal) for
// int8, the default for int4 (measured at K=4096, N=14336, M=1: int8 24.1 -> 23.4 us, int4 19.5 ->
// 21.2 us with sc0 nt).
template <bool I8>
constexpr int kSpPol = I8 ? 3 : 0;

template <bool I8, int C, int W, int P, bool XL>
__global__ __launch_bounds__(W * 64) void matvec_kernel(const _Float16* __restrict__ x, const uint8_t* __restrict__ Wt,
                                                        const _Float16* __restrict__ Ws, _Float16* __restrict__ y,
                                                        int M, int N, int K) {
  constexpr int TW = 16 * C;
  constexpr int kRedFloats = W * 8 * TW;
  constexpr int kLdsFloats = kRedFloats > kXsMax / 2 ? kRedFloats : kXsMax / 2;
  __shared__ __attribute__((aligned(16))) float lds[kLdsFloats];  // x staging, then the wave sums
  _Float16* xs = reinterpret_cast<_Float16*>(lds);
  float(*red)[8][TW] = reinterpret_cast<float(*)[8][TW]>(lds);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, q = lane >> 4;
  // Workgroups go to the 8 XCDs round-robin by id. A strip narrower than a 128-byte line of a
  // weight row (int4 here: 64 bytes) shares its lines with a neighbour, so the id is then remapped
  // to give each XCD a contiguous range of strips and both halves of a line are fetched into the
  // same L2 (in id order every int4 weight line went to two L2s; the remap measured 2% faster there
  // and 2% slower on int8's whole-line strips, which keep the id order).
  int strip = (int)blockIdx.x;
  if constexpr ((I8 ? C : C / 2) < 128 / 16) {
    const int nwg = (int)gridDim.x, xcd = strip & 7, idx = strip >> 3, qq = nwg >> 3, rr = nwg & 7;
    strip = (xcd < rr ? xcd * (qq + 1) : rr * (qq + 1) + (xcd - rr) * qq) + idx;
  }
  const int kb0 = 0, kb1 = K / 32;
  const int KC = K;
  const int n0 = strip * TW, col = n0 + C * i;

  if constexpr (XL) {  // activations x[m][0 .. K) -> xs[m*K + ...]
    for (int e = 8 * threadIdx.x; e < M * KC; e += 8 * W * 64) {
      const int m = e / KC, kk = e - m * KC;
      *reinterpret_cast<uint4*>(&xs[e]) = *reinterpret_cast<const uint4*>(x + (int64_t)m * K + 32 * kb0 + kk);
    }
  }
  // N is a multiple of C, so a lane's columns are all in or all out; lanes past N load the last
  // C columns, lanes past M the last activation row: their results are never stored.
  const uint32_t cl = (uint32_t)(col < N ? col : N - C);
  const int xrow = i < M ? i : M - 1;
  LaneOffsets lo;
  lo.w = I8 ? 8u * q * (uint32_t)N + cl : (8u * q * (uint32_t)N + cl) / 2u;
  lo.x = 2u * ((uint32_t)xrow * (uint32_t)K + 8u * q);
  lo.s = 2u * cl;
  lo.xt = 0;
  const rsrc_t xr = make_rsrc(x, XL ? 0u : 2u * (uint32_t)M * (uint32_t)K);
  const _Float16* xl = xs + xrow * KC + 8 * q;  // XL: + 32*(blk - kb0) is the lane's x fragment

  v4f acc[C];
#pragma unroll
  for (int j = 0; j < C; j++) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
  if constexpr (XL) __syncthreads();

  // this wave's blocks: kb0 + wave + W*u, u < cnt
  const int cnt = kb1 - kb0 > wave ? (kb1 - kb0 - wave + W - 1) / W : 0;
  auto blk = [&](int u) { return kb0 + wave + W * u; };
  auto xfrag = [&](const Stage<I8, C>& st, int u) {
    if constexpr (XL) return *reinterpret_cast<const v8h*>(xl + 32 * (wave + W * u));
    else return __builtin_bit_cast(v8h, st.xa[0]);
  };
  Stage<I8, C> ring[P];
  int t = 0;
  if (cnt >= 2 * P) {
    // Steady state: every slot is computed and refilled in order, with no conditions, so the
    // loads of a slot are always followed by those of the other P-1 slots and each compute waits
    // only for its own slot's loads.
#pragma unroll
    for (int s = 0; s < P; s++) {
      load_stage<I8, C, !XL, 1, kSpPol<I8>>(ring[s], Wt, xr, Ws, (uint32_t)N, blk(s), lo);
      __builtin_amdgcn_sched_barrier(0);
    }
    do {
#pragma unroll
      for (int s = 0; s < P; s++) {
        compute_stage<I8, C>(ring[s], xfrag(ring[s], t + s), acc);
        load_stage<I8, C, !XL, 1, kSpPol<I8>>(ring[s], Wt, xr, Ws, (uint32_t)N, blk(t + s + P), lo);
        // keep the refill here: left alone, the scheduler sinks every refill below all P computes
        __builtin_amdgcn_sched_barrier(0);
      }
      t += P;
    } while (t + 2 * P <= cnt);
  } else {
#pragma unroll
    for (int s = 0; s < P; s++)
      if (s < cnt) load_stage<I8, C, !XL, 1, kSpPol<I8>>(ring[s], Wt, xr, Ws, (uint32_t)N, blk(s), lo);
  }
  // drain: fewer than 2P blocks left, the first P of them (those < cnt) already in the ring
#pragma unroll
  for (int s = 0; s < P; s++) {
    if (t + s < cnt) {
      compute_stage<I8, C>(ring[s], xfrag(ring[s], t + s), acc);
      if (t + s + P < cnt) load_stage<I8, C, !XL, 1, kSpPol<I8>>(ring[s], Wt, xr, Ws, (uint32_t)N, blk(t + s + P), lo);
    }
  }
#pragma unroll
  for (int s = 0; s < P; s++)
    if (t + P + s < cnt) compute_stage<I8, C>(ring[s], xfrag(ring[s], t + P + s), acc);

  // acc[j][v] = this wave's share of y[4q+v][col+j]; rows >= M and columns >= N are dropped.
  if constexpr (XL) __syncthreads();  // every wave is done with xs before red overwrites it
  if (q < 2) {
#pragma unroll
    for (int j = 0; j < C; j++)
#pragma unroll
      for (int v = 0; v < 4; v++) red[wave][4 * q + v][C * i + j] = acc[j][v];
  }
  __syncthreads();
  for (int o = threadIdx.x; o < M * TW; o += W * 64) {
    const int m = o / TW, c = o % TW;
    if (n0 + c >= N) continue;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < W; w++) v += red[w][m][c];
    y[(int64_t)m * N + n0 + c] = (_Float16)v;
  }
}

// ---------------------------------------------------------------------------------------------
// Small-M GEMM form (9 <= M <= 256 activation rows: the same block-scaled product at prefill-like
// shapes). A workgroup owns MT tiles of 16 activation rows and a strip of TW = 16*C columns over
// the whole of K; its W waves split K as in the single-pass kernel. Each dequantised weight
// fragment of a block feeds MT MFMAs, one per activation tile, so the weight conversion is shared
// by 16*MT rows; every block product is still scaled by its fp16 block scale in fp32 (one FMA per
// output per block) and added to an fp32 accumulator. The waves' accumulators meet in LDS. Given a
// workspace, grids of few tiles also split K across workgroups (wq_split_plan below).
// ---------------------------------------------------------------------------------------------
// One block, software-pipelined across the column offsets e of the lane's C columns: the MFMAs of
// offset e (one per activation tile) alternate with the scale FMAs of offset e-1, whose products
// were issued a full round of MFMAs earlier, so neither the matrix core nor the vector ALU waits
// on the other. Each group of 4 columns is converted just before its first MFMA. The products of
// the last offset stay pending and are scaled during the first MFMA round of the next block;
// flush_pending() scales what the last block left. The full scheduling barriers keep this issue
// order (left alone, the scheduler puts each FMA right behind the MFMA that produces its input).
template <int MT>
struct Pending {
  v4f d[MT];   // products of the last column offset (column C-1) of the previous block
  uint32_t s;  // its fp16 scale (low half)
};

template <int C, int MT>
MX_DEV void scale_add(v4f (&acc)[MT][C], const v4f& d, int t, int j, uint32_t sh) {
  const float sj = (float)as_v2h(sh)[0];
#pragma unroll
  for (int v = 0; v < 4; v++) acc[t][j][v] = __builtin_fmaf(sj, d[v], acc[t][j][v]);
}

template <bool I8, int C, int MT>
MX_DEV void compute_stage_mt(const Stage<I8, C, MT>& s, v4f (&acc)[MT][C], Pending<MT>& pend) {
  static_assert(C % 4 == 0, "groups of 4 columns per lane");
  v8h frag[4];
  v4f d[2][MT];
#pragma unroll
  for (int e = 0; e < C; e++) {
    if (e % 4 == 0) {
      weights_to_frags<I8, C>(s, e / 4, frag);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < MT; t++) {
      d[e & 1][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, s.xa[t]), frag[e % 4],
                                                           v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      if (e == 0) scale_add<C, MT>(acc, pend.d[t], t, C - 1, pend.s);
      else scale_add<C, MT>(acc, d[(e - 1) & 1][t], t, e - 1, (e - 1) & 1 ? s.sc[(e - 1) / 2] >> 16 : s.sc[(e - 1) / 2]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int t = 0; t < MT; t++) pend.d[t] = d[(C - 1) & 1][t];
  pend.s = (C - 1) & 1 ? s.sc[(C - 1) / 2] >> 16 : s.sc[(C - 1) / 2];
}

template <int C, int MT>
MX_DEV void flush_pending(v4f (&acc)[MT][C], const Pending<MT>& pend) {
#pragma unroll
  for (int t = 0; t < MT; t++) scale_add<C, MT>(acc, pend.d[t], t, C - 1, pend.s);
}

constexpr int kWqWPol = 0;  // cache policy of the weight and scale loads
constexpr int kWqMaxSplits = 8;  // K splits of the small-M GEMM, and workgroups sharing a tile

// Each workgroup takes one run of 32-row blocks out of the sequence of all tiles' blocks (tile
// after tile, K order within a tile) and walks it tile by tile:
// - S > 1 (grid.y = S, QB = 0): K is split, workgroup (tile, sk) takes the blocks
//   [sk nblk / S, (sk + 1) nblk / S) of its tile and writes its fp32 partial tile to
//   part[sk][M][N].
// - RUNS (grid.y = 1, one workgroup per CU): the sequence is dealt out in equal runs of QB
//   blocks, workgroup w taking [w QB, (w + 1) QB), so every workgroup has the same work however the
//   tile count falls against the CU count. A run may end inside a tile and the next run go on in
//   it; a tile wholly inside one run is stored directly. A run ends in at most two shared tiles
//   (its first and its last), whose fp32 partial tiles go to slots 2w and 2w + 1 of
//   part[slot][16 MT][16 C].
// The workgroups that share a tile (its contributors, in run order) store their partials, and the
// last to arrive adds them in run order (the same protocol as the split matvec below:
// system-coherent 16-byte stores acknowledged before a device-scope counter increment on
// counters[tile], which the last workgroup takes from (contributors - 1) back to 0).
// Waves per SIMD the compiler must allow: two workgroups per CU for the 8-wave shapes of 4 columns
// per lane with at most 32-row tiles (the split epilogue otherwise makes it settle for one workgroup
// and twice the registers).
template <int C, int MT, int W>
constexpr int wq_waves_per_eu() { return C == 4 && W == 8 && MT <= 2 ? 4 : W / 4; }

template <bool I8, int C, int MT, int W, int P, bool RUNS>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(wq_waves_per_eu<C, MT, W>())))
void gemm_wq_kernel(const _Float16* __restrict__ x, const uint8_t* __restrict__ Wt,
                                                         const _Float16* __restrict__ Ws, _Float16* __restrict__ y,
                                                         int M, int N, int K, float* __restrict__ part,
                                                         unsigned* __restrict__ counters, int S, int QB) {
  constexpr int TW = 16 * C, RT = 16 * MT;  // columns and activation rows of the workgroup's tile
  __shared__ __attribute__((aligned(16))) float red[W][RT][TW];
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, q = lane >> 4;
  // Workgroups go to the 8 XCDs (each with its own L2) round-robin by id. A strip is 16*C columns,
  // less than a 128-byte line of a weight row (32 bytes for int4), so neighbouring strips share
  // lines: the id is remapped so that each XCD takes a contiguous range of (strip, row tile) pairs,
  // row tiles fastest, and every line is fetched into one L2 only.
  const int nwg = (int)gridDim.x, mtiles = (M + RT - 1) / RT;
  int bid = (int)blockIdx.x;
  {
    const int xcd = bid & 7, idx = bid >> 3, qq = nwg >> 3, rr = nwg & 7;
    bid = (xcd < rr ? xcd * (qq + 1) : rr * (qq + 1) + (xcd - rr) * qq) + idx;
  }
  const int sk = (int)blockIdx.y, nall = K / 32;
  const int64_t nseq = (int64_t)mtiles * ((N + TW - 1) / TW) * nall;
  int64_t g, gend;  // this workgroup's run [g, gend) of the block sequence
  if (RUNS) {
    g = (int64_t)bid * QB;
    gend = g + QB < nseq ? g + QB : nseq;
  } else {
    g = (int64_t)bid * nall + (int64_t)sk * nall / S;
    gend = (int64_t)bid * nall + (int64_t)(sk + 1) * nall / S;
  }

#pragma unroll 1
  for (;;) {
    const int tile = (int)(g / nall), kb0 = (int)(g - (int64_t)tile * nall);
    const int64_t tbeg = (int64_t)tile * nall, tend = tbeg + nall;
    const int nblk = (int)((gend < tend ? gend : tend) - g);
    int first = 0, nc = S;  // the tile's first contributor and their number
    if (RUNS) {
      first = (int)(tbeg / QB);
      nc = (int)((tend - 1) / QB) - first + 1;
    }
    const int n0 = (tile / mtiles) * TW, m0 = (tile % mtiles) * RT, col = n0 + C * i;

    // Columns as in the single-pass kernel (lanes past N load the last C columns). Activation rows
    // come through a resource over rows m0..M-1: rows past M read as zero, their outputs are dropped.
    const uint32_t cl = (uint32_t)(col < N ? col : N - C);
    LaneOffsets lo;
    lo.w = I8 ? 8u * q * (uint32_t)N + cl : (8u * q * (uint32_t)N + cl) / 2u;
    lo.x = 2u * ((uint32_t)i * (uint32_t)K + 8u * q);
    lo.s = 2u * cl;
    lo.xt = 32u * (uint32_t)K;
    const rsrc_t xr = make_rsrc(x + (int64_t)m0 * K, 2u * (uint32_t)(M - m0) * (uint32_t)K);

    v4f acc[MT][C];
#pragma unroll
    for (int t = 0; t < MT; t++)
#pragma unroll
      for (int j = 0; j < C; j++) acc[t][j] = v4f{0.f, 0.f, 0.f, 0.f};
    Pending<MT> pend;  // nothing pending yet: zero products (adding +0 leaves the +0 accumulators)
#pragma unroll
    for (int t = 0; t < MT; t++) pend.d[t] = v4f{0.f, 0.f, 0.f, 0.f};
    pend.s = 0;

    // this wave's blocks: wave + W*u, u < cnt; loads run P blocks ahead through a register ring
    const int cnt = nblk > wave ? (nblk - wave + W - 1) / W : 0;
    auto blk = [&](int u) { return kb0 + wave + W * u; };
    Stage<I8, C, MT> ring[P];
    int t = 0;
    if (cnt >= 2 * P) {
#pragma unroll
      for (int s = 0; s < P; s++) {
        load_stage<I8, C, true, MT, kWqWPol>(ring[s], Wt, xr, Ws, (uint32_t)N, blk(s), lo);
        __builtin_amdgcn_sched_barrier(0);
      }
      do {
#pragma unroll
        for (int s = 0; s < P; s++) {
          compute_stage_mt<I8, C, MT>(ring[s], acc, pend);
          load_stage<I8, C, true, MT, kWqWPol>(ring[s], Wt, xr, Ws, (uint32_t)N, blk(t + s + P), lo);
          __builtin_amdgcn_sched_barrier(0);
        }
        t += P;
      } while (t + 2 * P <= cnt);
    } else {
#pragma unroll
      for (int s = 0; s < P; s++)
        if (s < cnt) load_stage<I8, C, true, MT, kWqWPol>(ring[s], Wt, xr, Ws, (uint32_t)N, blk(s), lo);
    }
#pragma unroll
    for (int s = 0; s < P; s++) {
      if (t + s < cnt) {
        compute_stage_mt<I8, C, MT>(ring[s], acc, pend);
        if (t + s + P < cnt) load_stage<I8, C, true, MT, kWqWPol>(ring[s], Wt, xr, Ws, (uint32_t)N, blk(t + s + P), lo);
      }
    }
#pragma unroll
    for (int s = 0; s < P; s++)
      if (t + P + s < cnt) compute_stage_mt<I8, C, MT>(ring[s], acc, pend);

    flush_pending<C, MT>(acc, pend);
    // acc[t][j][v] = this wave's share of y[m0 + 16t + 4q + v][col + j]
#pragma unroll
    for (int tt = 0; tt < MT; tt++)
#pragma unroll
      for (int j = 0; j < C; j++)
#pragma unroll
        for (int v = 0; v < 4; v++) red[wave][16 * tt + 4 * q + v][C * i + j] = acc[tt][j][v];
    __syncthreads();
    const int rows = min(RT, M - m0);
    if (nc == 1) {
      for (int o = threadIdx.x; o < rows * (TW / 4); o += W * 64) {
        const int r = o / (TW / 4), c = 4 * (o % (TW / 4));
        if (n0 + c >= N) continue;  // N % 4 == 0: a 4-column group is all in or all out
        v4f v = *reinterpret_cast<const v4f*>(&red[0][r][c]);
#pragma unroll
        for (int w = 1; w < W; w++) v += *reinterpret_cast<const v4f*>(&red[w][r][c]);
        v4h h;
#pragma unroll
        for (int e = 0; e < 4; e++) h[e] = (_Float16)v[e];
        *reinterpret_cast<v4h*>(y + (int64_t)(m0 + r) * N + n0 + c) = h;
      }
    } else {
      // byte offset of element (r, c) of contributor j's partial tile
      auto poff = [&](int j, int r, int c) -> uint32_t {
        if (RUNS) {
          const int w = first + j;
          const int slot = 2 * w + ((int64_t)w * QB >= tbeg ? 0 : 1);  // the run's first or last tile
          return 4u * (uint32_t)((slot * RT + r) * TW + c);
        }
        return 4u * (uint32_t)(((j * M) + m0 + r) * N + n0 + c);
      };
      const uint32_t pbytes = RUNS ? 8u * (uint32_t)nwg * RT * TW : 4u * (uint32_t)S * (uint32_t)M * (uint32_t)N;
      const rsrc_t pr = make_rsrc(part, pbytes);
      const int jc = RUNS ? bid - first : sk;
#pragma unroll 1
      for (int o = threadIdx.x; o < rows * (TW / 4); o += W * 64) {
        const int r = o / (TW / 4), c = 4 * (o % (TW / 4));
        if (n0 + c >= N) continue;
        v4f v = *reinterpret_cast<const v4f*>(&red[0][r][c]);
#pragma unroll
        for (int w = 1; w < W; w++) v += *reinterpret_cast<const v4f*>(&red[w][r][c]);
        // element copies first: a bit cast of an ext-vector element read element 0
        const float e0 = v[0], e1 = v[1], e2 = v[2], e3 = v[3];
        const u4 val = {__builtin_bit_cast(uint32_t, e0), __builtin_bit_cast(uint32_t, e1),
                        __builtin_bit_cast(uint32_t, e2), __builtin_bit_cast(uint32_t, e3)};
        __builtin_amdgcn_raw_buffer_store_b128(val, pr, poff(jc, r, c), 0, 17);  // sc0 sc1
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's partial stores are acknowledged
      __syncthreads();
      // the flag lives in red, free once every thread is past its reads above (an extra LDS variable
      // would cost this kernel its occupancy: the compiler rounds the allocation up)
      int* last = reinterpret_cast<int*>(&red[0][0][0]);
      if (threadIdx.x == 0) *last = atomicInc(&counters[tile], (unsigned)(nc - 1)) == (unsigned)(nc - 1);
      __syncthreads();
      if (*last) {
#pragma unroll 1
        for (int o = threadIdx.x; o < rows * (TW / 4); o += W * 64) {
          const int r = o / (TW / 4), c = 4 * (o % (TW / 4));
          if (n0 + c >= N) continue;
          u4 v[kWqMaxSplits];
#pragma unroll
          for (int sp = 0; sp < kWqMaxSplits; sp++)
            if (sp < nc) v[sp] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(pr, poff(sp, r, c), 0, 17));
          float sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int sp = 0; sp < kWqMaxSplits; sp++)
            if (sp < nc) {
              const u4 w = v[sp];
              const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
              sum[0] += __builtin_bit_cast(float, w0);
              sum[1] += __builtin_bit_cast(float, w1);
              sum[2] += __builtin_bit_cast(float, w2);
              sum[3] += __builtin_bit_cast(float, w3);
            }
          v4h h;
#pragma unroll
          for (int e = 0; e < 4; e++) h[e] = (_Float16)sum[e];
          *reinterpret_cast<v4h*>(y + (int64_t)(m0 + r) * N + n0 + c) = h;
        }
      }
    }
    g += nblk;
    if (!RUNS || g >= gend) break;
    __syncthreads();  // red, and the flag in it, are written again for the next tile
  }
}

constexpr int kMaxSplits = 16;

// ---------------------------------------------------------------------------------------------
// Split-K kernel with LDS staging. HBM streams best when a load instruction covers long runs of
// bytes (16 bytes per lane, whole 128-byte lines); the MFMA operand layout wants 8 rows of a few
// adjacent columns per lane. Direct global->LDS loads decouple the two:
//  - A workgroup (8 waves) owns a strip of 64*CG bytes of every row (int8: CG = 4, 256 columns;
//    int4: CG = 2, 256 columns) and the 32-row blocks [kb0, kb1) of its K split.
//  - A stage is one block: 1 KB chunks of CR rows (4 rows x 256 bytes or 8 rows x 128 bytes) plus
//    the block's scale row, copied straight into an R-stage LDS ring. Chunks are padded (1056 or
//    1088 bytes), so the fragment reads below hit 4 disjoint bank groups.
//  - Waves (cg, par), cg < CG, par < PAR = 8 / CG: a step is PAR stages; the waves of parity par
//    compute stage PAR u + par of step u, wave cg the strip's columns [16*C*cg, 16*C*(cg+1)) (64
//    bytes of each row). Lane (i, q) reads the dword of rows 8q..8q+7 holding its C columns,
//    exactly the register layout of the single-pass kernel, and the same convert / MFMA / scale
//    code runs.
//  - The activations of the split's K range sit in LDS (staged once).
// ---------------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_ptr_t;
constexpr int kXsLds = 8192;                 // activation halfs staged per workgroup

// Geometry of the split kernel with CG column groups of 64 bytes per row: a strip is 64*CG bytes of
// every row (TW columns), a copy instruction fills a 1 KB chunk of CR rows, a 32-row block is NCH
// chunks (padded to LCH bytes, so the fragment reads of the 4 row groups q hit disjoint bank
// groups) plus its scale row, and the 8 waves are CG column groups x PAR stage parities.
template <bool I8, int CG>
struct LdsGeo {
  static constexpr int C = I8 ? 4 : 8;        // columns per lane
  static constexpr int TW = 16 * C * CG;      // columns per strip
  static constexpr int SBYTES = 64 * CG;      // bytes of a row in the strip
  static constexpr int PAR = 8 / CG;          // stages (32-row blocks) per step
  static constexpr int CR = 1024 / SBYTES;    // rows per chunk
  static constexpr int NCH = 32 / CR;         // chunks per block (= 2 CG: wave (cg, par) copies 2cg, 2cg+1)
  static constexpr int LCH = 1024 + 256 / NCH;  // padded chunk stride
  static constexpr int SB = 2 * TW;           // scale bytes of a strip row
  static constexpr int STAGE = NCH * LCH + 1024;  // the scale row (SB <= 1 KB) in a whole 1 KB
  static constexpr int SLANES = SB / CG / 16;  // lanes per wave copying scales
  // LDS offset of row j (0..7) of the lane's 8 fragment rows from its first row's dword
  static constexpr int roff(int j) { return (j / CR) * LCH + (j % CR) * SBYTES; }
  static_assert(CG == 2 || CG == 4, "strips of 128 or 256 bytes per row");
  static_assert(NCH == 2 * CG && (LCH / 4) * (8 / CR) % 64 == 16 && SB <= 1024, "copy split and bank layout");
};
static_assert(kXsLds % 512 == 0, "the activation copies fill whole 1 KB pieces of xs");

// vmcnt(n) with the other counters left alone (gfx9 s_waitcnt encoding)
MX_DEV void wait_vm_n(int n) {
  switch (n) {
#define MX_W(k) \
  case k: __builtin_amdgcn_s_waitcnt(((k) & 0xF) | 0x0F70 | ((((k) >> 4) & 3) << 14)); break;
    MX_W(0) MX_W(1) MX_W(2) MX_W(3) MX_W(4) MX_W(5) MX_W(6) MX_W(7) MX_W(8) MX_W(9) MX_W(10) MX_W(11)
    MX_W(12) MX_W(13) MX_W(14) MX_W(15) MX_W(16) MX_W(17) MX_W(18) MX_W(19) MX_W(20) MX_W(21)
#undef MX_W
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
}
// Workgroup barrier without the fences of __syncthreads() (which would wait for every queued
// direct copy); the waits the ring needs are explicit.
MX_DEV void raw_barrier() { asm volatile("s_barrier" ::: "memory"); }
MX_DEV void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0) only

// The lane's 8 fragment dwords (rows 8q..8q+7 of a stage, at the geometry's row offsets) and its C
// scales, read from the ring with one lgkmcnt wait. Written as inline
// assembly because the compiler cannot tell these reads from the ring slot that the direct copies
// queued just before are filling, and would otherwise wait for every queued copy (vmcnt(0)) here.
// The outputs are early-clobber: a read's destination must not be an address register of a later
// read in the block (its data may land before that read issues).
template <bool I8, int CG>
MX_DEV void read_stage(Stage<I8, LdsGeo<I8, CG>::C>& sg, uint32_t aw, uint32_t as) {
  using G = LdsGeo<I8, CG>;
  static_assert(Stage<I8, G::C>::kWordsPerRow == 1, "one dword per row and lane");
  if constexpr (G::C == 4) {
    uint64_t sc;
    asm volatile(
        "ds_read_b32 %0, %9 offset:%11\n"
        "ds_read_b32 %1, %9 offset:%12\n"
        "ds_read_b32 %2, %9 offset:%13\n"
        "ds_read_b32 %3, %9 offset:%14\n"
        "ds_read_b32 %4, %9 offset:%15\n"
        "ds_read_b32 %5, %9 offset:%16\n"
        "ds_read_b32 %6, %9 offset:%17\n"
        "ds_read_b32 %7, %9 offset:%18\n"
        "ds_read_b64 %8, %10\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(sg.w[0][0]), "=&v"(sg.w[1][0]), "=&v"(sg.w[2][0]), "=&v"(sg.w[3][0]), "=&v"(sg.w[4][0]),
          "=&v"(sg.w[5][0]), "=&v"(sg.w[6][0]), "=&v"(sg.w[7][0]), "=&v"(sc)
        : "v"(aw), "v"(as), "i"(G::roff(0)), "i"(G::roff(1)), "i"(G::roff(2)), "i"(G::roff(3)), "i"(G::roff(4)),
          "i"(G::roff(5)), "i"(G::roff(6)), "i"(G::roff(7)));
    sg.sc[0] = (uint32_t)sc;
    sg.sc[1] = (uint32_t)(sc >> 32);
  } else {
    static_assert(G::C == 8, "4 or 8 columns per lane");
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    u4 sc;
    asm volatile(
        "ds_read_b32 %0, %9 offset:%11\n"
        "ds_read_b32 %1, %9 offset:%12\n"
        "ds_read_b32 %2, %9 offset:%13\n"
        "ds_read_b32 %3, %9 offset:%14\n"
        "ds_read_b32 %4, %9 offset:%15\n"
        "ds_read_b32 %5, %9 offset:%16\n"
        "ds_read_b32 %6, %9 offset:%17\n"
        "ds_read_b32 %7, %9 offset:%18\n"
        "ds_read_b128 %8, %10\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(sg.w[0][0]), "=&v"(sg.w[1][0]), "=&v"(sg.w[2][0]), "=&v"(sg.w[3][0]), "=&v"(sg.w[4][0]),
          "=&v"(sg.w[5][0]), "=&v"(sg.w[6][0]), "=&v"(sg.w[7][0]), "=&v"(sc)
        : "v"(aw), "v"(as), "i"(G::roff(0)), "i"(G::roff(1)), "i"(G::roff(2)), "i"(G::roff(3)), "i"(G::roff(4)),
          "i"(G::roff(5)), "i"(G::roff(6)), "i"(G::roff(7)));
    sg.sc[0] = sc[0];
    sg.sc[1] = sc[1];
    sg.sc[2] = sc[2];
    sg.sc[3] = sc[3];
  }
}

template <bool I8, int R, int CG, bool M1>
__global__ __launch_bounds__(512) void matvec_lds_kernel(const _Float16* __restrict__ x, const uint8_t* __restrict__ Wt,
                                                         const _Float16* __restrict__ Ws, _Float16* __restrict__ y,
                                                         float* __restrict__ part, unsigned* __restrict__ counters,
                                                         int M, int N, int K, int S) {
  using G = LdsGeo<I8, CG>;
  constexpr int C = G::C, TW = G::TW, SB = G::SB, PAR = G::PAR, STAGE = G::STAGE;
  constexpr int kLoads = 3;                           // direct copies per wave per step
  constexpr int RS = R / PAR;                         // ring slots of PAR stages (a step)
  static_assert(R % PAR == 0 && RS >= 2 && kLoads * (RS - 2) <= 21, "wait_vm_n range");
  static_assert(R * STAGE >= (PAR - 1) * CG * 64 * 4 * C * 4, "the other parities' sums fit in the ring");
  __shared__ __attribute__((aligned(16))) char ring[R * STAGE];
  __shared__ __attribute__((aligned(16))) _Float16 xs[kXsLds];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cg = wave % CG, par = wave / CG;  // column group, stage parity
  const int i = lane & 15, q = lane >> 4;
  const int strip = blockIdx.x, sk = blockIdx.y, nblk = K / 32;
  const int kb0 = (int)((int64_t)sk * nblk / S), kb1 = (int)((int64_t)(sk + 1) * nblk / S);
  const int nb = kb1 - kb0, KC = 32 * nb, nsteps = (nb + PAR - 1) / PAR;
  const int n0 = strip * TW, col = n0 + 16 * C * cg + C * i;
  const uint32_t row_bytes = I8 ? (uint32_t)N : (uint32_t)N / 2;

  // Activations x[m][32*kb0 .. 32*kb1) -> xs[m*KC + ...] as direct copies queued ahead of the
  // ring's, so the first step's wait covers them: copy j (from wave j % 8) fills xs halfs
  // 512j .. 512j+511, lane l the 8 from 512j + 8l. Lanes past M*KC re-read x's first 16 bytes into
  // unused xs (M*KC <= kXsLds, a multiple of 512, so every copy stays inside xs).
  {
    const rsrc_t xr = make_rsrc(x, 2u * (uint32_t)M * (uint32_t)K);
    const int nj = (M * KC + 511) / 512;
    for (int j = wave; j < nj; j += 8) {
      const int e = 512 * j + 8 * lane;
      const int m = e / KC, kk = e - m * KC;
      const uint32_t vo = e < M * KC ? 2u * (uint32_t)(m * K + 32 * kb0 + kk) : 0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(xs + 512 * j), 16, vo, 0, 0, 0);
    }
  }

  // Copy offsets: lane l of a chunk copy fills row l / LPR of the chunk, bytes 16 (l % LPR) of the
  // strip row (LPR = lanes per row). Bytes past the end of a row (last strip) are clamped back into
  // the row; the columns they feed are never stored. Row bytes and 2N are multiples of 16.
  constexpr uint32_t LPR = G::SBYTES / 16;
  uint32_t colb = (uint32_t)strip * G::SBYTES + 16u * ((uint32_t)lane % LPR);
  if (colb > row_bytes - 16u) colb = row_bytes - 16u;
  const uint32_t voff0 = ((uint32_t)G::CR * (2u * cg) + (uint32_t)lane / LPR) * row_bytes + colb;
  const uint32_t voff1 = voff0 + (uint32_t)G::CR * row_bytes;
  uint32_t scb = 2u * (uint32_t)n0 + (uint32_t)cg * (SB / CG) + 16u * (uint32_t)lane;
  if (scb > 2u * (uint32_t)N - 16u) scb = 2u * (uint32_t)N - 16u;

  // Step u: wave (cg, par) copies chunks 2cg, 2cg+1 and scale part cg of stage PAR u + par. A
  // stage past the split (a block count that is not a multiple of PAR) re-reads the split's last
  // block, so every wave queues the same number of copies per step and the vmcnt accounting stays
  // exact.
  auto issue = [&](int u) {
    const int stage = PAR * u + par, blk = kb0 + (stage < nb ? stage : nb - 1);
    char* st = ring + ((u % RS) * PAR + par) * STAGE;
    // weights and scales are read exactly once: past the CU's L1 (sc0) and non-temporal (nt) in the
    // L2 (measured 1-3% faster than the default policy at the decode shapes)
    const rsrc_t wr = make_rsrc(Wt + (int64_t)blk * 32 * row_bytes, 32u * row_bytes);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(st + (2 * cg) * G::LCH), 16, voff0, 0, 0, 3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(st + (2 * cg + 1) * G::LCH), 16, voff1, 0, 0, 3);
    const rsrc_t sr = make_rsrc(Ws + (int64_t)blk * N, 2u * (uint32_t)N);
    if (lane < G::SLANES)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_ptr_t)(st + G::NCH * G::LCH + cg * (SB / CG)), 16, scb, 0, 0,
                                               3);
  };

  const int xrow = i < M ? i : M - 1;
  const _Float16* xl = xs + xrow * KC + 8 * q;
  // LDS byte addresses of the lane's fragment dword (rows 8q.. of this parity's stage in ring
  // slot 0) and of its scales
  const uint32_t ring0 = (uint32_t)(uintptr_t)(lds_ptr_t)ring + (uint32_t)(par * STAGE);
  const uint32_t lds_w = ring0 + (uint32_t)((8 * q / G::CR) * G::LCH + cg * 64 + 4 * i);
  const uint32_t lds_s = ring0 + (uint32_t)(G::NCH * G::LCH + 2 * (16 * C * cg + C * i));
  v4f acc[C];
#pragma unroll
  for (int j = 0; j < C; j++) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int u = 0; u < RS - 1; u++)
    if (u < nsteps) issue(u);

  for (int u = 0; u < nsteps; u++) {
    const int after = nsteps - 1 - u < RS - 2 ? nsteps - 1 - u : RS - 2;  // steps queued after u
    wait_vm_n(kLoads * after);  // this wave's copies of step u have landed ...
    wait_lds();                 // ... and its reads of step u-1 are done
    raw_barrier();              // every wave: step u visible, slot (u-1)%RS free
    if (u + RS - 1 < nsteps) issue(u + RS - 1);
    if (PAR * u + par < nb) {
      Stage<I8, C> sg;
      const uint32_t so = (uint32_t)((u % RS) * PAR * STAGE);
      read_stage<I8, CG>(sg, lds_w + so, lds_s + so);
      compute_stage<I8, C, M1 ? 1 : 4>(sg, *reinterpret_cast<const v8h*>(xl + 32 * (PAR * u + par)), acc);
    }
  }

  // the parities' sums meet in LDS (the ring is free once every wave is past its last read): parity
  // p > 0 writes region p-1, parity 0 adds them in parity order
  wait_lds();
  raw_barrier();
  float* red = reinterpret_cast<float*>(ring) + (cg * 64 + lane) * (4 * C);
  constexpr int RSTRIDE = CG * 64 * 4 * C;  // floats per parity region
  if (par > 0) {
#pragma unroll
    for (int j = 0; j < C; j++) *reinterpret_cast<v4f*>(red + (par - 1) * RSTRIDE + 4 * j) = acc[j];
  }
  __syncthreads();
  if (par == 0) {
#pragma unroll
    for (int p = 1; p < PAR; p++)
#pragma unroll
      for (int j = 0; j < C; j++) acc[j] += *reinterpret_cast<const v4f*>(red + (p - 1) * RSTRIDE + 4 * j);
  }

  // acc[j][v] (parity-0 waves) = the split's y[4q+v][col+j]; rows >= M and columns >= N are
  // dropped.
  if (S == 1) {
    if (par == 0 && col < N) {
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int m = 4 * q + v;
        if (m < M) {
#pragma unroll
          for (int g = 0; g < C / 4; g++) {
            v4h o;
#pragma unroll
            for (int e = 0; e < 4; e++) o[e] = (_Float16)acc[4 * g + e][v];
            *reinterpret_cast<v4h*>(y + (int64_t)m * N + col + 4 * g) = o;
          }
        }
      }
    }
    return;
  }
  // Cross-split sum. Partial tiles live in the workspace as rows of Npad = NS * TW floats per split
  // and activation row, permuted within each strip so that every store instruction of a wave writes
  // 16 lanes x 16 contiguous bytes: column 16 C cg + C i + 4 g of the strip (lane i of column group
  // cg, its 4-column group g) sits at float ((cg (C/4) + g) 16 + i) 4 of the strip's row. The
  // stores and the loads below carry the system-coherence bits (sc0 sc1): stores are written
  // through to memory and loads bypass every cache that is not coherent across XCDs, as relaxed
  // system-scope atomic accesses are on gfx950. Ordering: every wave waits for its stores to be
  // acknowledged (vmcnt(0)) before the workgroup's barrier and the strip counter's increment (a
  // device-scope atomic); the workgroup that takes the counter from S-1 (back to 0) is the last,
  // every other one has incremented after its stores completed, so its loads see them all; it adds
  // the S partials in split order.
  const int Npad = (int)gridDim.x * TW;
  if (par == 0 && col < N) {
    const rsrc_t pr = make_rsrc(part, (uint32_t)S * (uint32_t)M * (uint32_t)Npad * 4u);
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const int m = 4 * q + v;
      if (m < M) {
#pragma unroll
        for (int g = 0; g < C / 4; g++) {
          const uint32_t off = 4u * (uint32_t)(((sk * M + m) * Npad) + n0 + ((cg * (C / 4) + g) * 16 + i) * 4);
          // element copies first: a bit cast of an ext-vector element read element 0 here
          const float e0 = acc[4 * g][v], e1 = acc[4 * g + 1][v], e2 = acc[4 * g + 2][v], e3 = acc[4 * g + 3][v];
          typedef uint32_t u4 __attribute__((ext_vector_type(4)));
          const u4 val = {__builtin_bit_cast(uint32_t, e0), __builtin_bit_cast(uint32_t, e1),
                          __builtin_bit_cast(uint32_t, e2), __builtin_bit_cast(uint32_t, e3)};
          __builtin_amdgcn_raw_buffer_store_b128(val, pr, off, 0, 17);  // sc0 sc1
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's partial stores are acknowledged
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomicInc(&counters[strip], (unsigned)(S - 1)) == (unsigned)(S - 1);
  __syncthreads();
  if (!s_last) return;
  // Each thread sums up to two 4-column groups (M * TW / 4 <= 1024 = 2 * 512), with every split's
  // 16-byte load of both groups in flight at once, in split order.
  {
    constexpr int kG = 2;
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    const rsrc_t pr = make_rsrc(part, (uint32_t)S * (uint32_t)M * (uint32_t)Npad * 4u);
    u4 v[kG][kMaxSplits];
    int og[kG];
#pragma unroll
    for (int g = 0; g < kG; g++) {
      const int o = 4 * (threadIdx.x + 512 * g), m = o / TW, cl = o - m * TW, c = n0 + cl;
      og[g] = (o < M * TW && c < N) ? o : -1;
      if (og[g] < 0) continue;
      // storage position of column cl of the strip: cl = 16 C cg + C i + 4 gg
      const int cg2 = cl / (16 * C), rem = cl - cg2 * 16 * C, i2 = rem / C, g2 = (rem - i2 * C) / 4;
      const int pos = ((cg2 * (C / 4) + g2) * 16 + i2) * 4;
#pragma unroll
      for (int sp = 0; sp < kMaxSplits; sp++)
        if (sp < S)
          v[g][sp] = __builtin_bit_cast(
              u4, __builtin_amdgcn_raw_buffer_load_b128(pr, 4u * (uint32_t)((sp * M + m) * Npad + n0 + pos), 0, 17));
    }
#pragma unroll
    for (int g = 0; g < kG; g++) {
      if (og[g] < 0) continue;
      const int o = og[g], m = o / TW, c = n0 + (o - m * TW);
      float sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sp = 0; sp < kMaxSplits; sp++)
        if (sp < S) {
          const u4 w = v[g][sp];
          const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
          sum[0] += __builtin_bit_cast(float, w0);
          sum[1] += __builtin_bit_cast(float, w1);
          sum[2] += __builtin_bit_cast(float, w2);
          sum[3] += __builtin_bit_cast(float, w3);
        }
      v4h h;
#pragma unroll
      for (int e = 0; e < 4; e++) h[e] = (_Float16)sum[e];
      *reinterpret_cast<v4h*>(y + (int64_t)m * N + c) = h;
    }
  }
}

// Single-pass kernel shape (no workspace): 8 columns per lane (a strip is 128 bytes of every int8
// row, 64 of every int4 row); 8 waves per workgroup, 4 (int8) or 2 (int4) blocks of loads in flight
// per wave. Measured at K=4096, N=14336: int4 with 16 columns per lane (128-byte rows, but only 56
// workgroups) 25.3 us at M=1, with 8 columns and 2 blocks ahead 19.6 us (3 or 4 ahead: 20.1-20.2,
// 4 columns: 22.8); int8 with 4 columns (224 workgroups of 64-byte rows) 24.3 against 24.1 us.
constexpr int kC8 = 8, kC4 = 8, kW = 8, kP8 = 4, kP4 = 2;
// Split kernel: strips of 256 bytes of every row (4 column groups) for int8 and 128 bytes (2 column
// groups, 4 stage parities) for int4, with rings of 8 and 12 stages (4 and 3 steps); K is split
// until about kTargetWGs workgroups run. int4 had 512-column strips (256 bytes) with 9 splits at
// N=14336, whose last workgroup read 9 partial tiles of M x 512 floats alone: 16.5 us at M=8
// against 14.4 us now (13.3 us at M=1 both ways). int4 rings of 16 / 20 / 24 stages measured 1-6%
// slower than 12.
constexpr int kCG8 = 4, kCG4 = 2, kR8 = 8, kR4 = 12, kTargetWGs = 256;

// Workspace layout: a fixed counter region (one counter per column strip, room for the largest
// strip count any shape can have), then the fp32 partials [S][M][NS * TW] (strips permuted, see the
// split kernel). Counters never share bytes
// with partials of any shape, so a workspace whose counters one call left at zero is valid for
// every later call.
constexpr size_t kCounterBytes = 16384;
static_assert(kCounterBytes / 4 >= MX_MAX_DIM / 256, "a counter per int8 strip of the widest matrix");

struct SplitPlan {
  int S, NS;     // K splits, column strips of the split kernel (S == 1: single-pass kernel)
  size_t bytes;  // workspace bytes (0 when S == 1)
};

SplitPlan split_plan(int M, int N, int K, bool int8) {
  const int tw = int8 ? LdsGeo<true, kCG8>::TW : LdsGeo<false, kCG4>::TW, nblk = K / 32;
  SplitPlan p;
  p.NS = (N + tw - 1) / tw;
  int S = kTargetWGs / p.NS;
  if (S > kMaxSplits) S = kMaxSplits;
  if (S > nblk / 4) S = nblk / 4;  // at least 4 blocks per split
  if (S < 2) {                     // not worth splitting: single pass
    p.S = 1;
    p.bytes = 0;
    return p;
  }
  while (M * 32 * ((nblk + S - 1) / S) > kXsLds) S++;  // the split's activations fit in LDS
  if (S > kMaxSplits) {                                 // too many: single pass
    p.S = 1;
    p.bytes = 0;
    return p;
  }
  p.S = S;
  p.bytes = kCounterBytes + (size_t)S * M * ((size_t)p.NS * tw) * 4;  // partial rows padded to whole strips
  return p;
}

template <bool I8>
int launch(int M, int N, int K, const void* x, const void* W, const void* Ws, void* y, void* ws, size_t ws_bytes,
           hipStream_t st) {
  const SplitPlan sp = split_plan(M, N, K, I8);
  if (sp.S > 1 && ws && ws_bytes >= sp.bytes) {
    unsigned* counters = (unsigned*)ws;
    float* part = (float*)((char*)ws + kCounterBytes);
    // M = 1 scales only output row 0 of each block product (1.6% / 2.6% faster at int8 / int4)
    if (M == 1)
      hipLaunchKernelGGL((matvec_lds_kernel<I8, I8 ? kR8 : kR4, I8 ? kCG8 : kCG4, true>),
                         dim3((unsigned)sp.NS, (unsigned)sp.S), dim3(512), 0, st, (const _Float16*)x, (const uint8_t*)W,
                         (const _Float16*)Ws, (_Float16*)y, part, counters, M, N, K, sp.S);
    else
      hipLaunchKernelGGL((matvec_lds_kernel<I8, I8 ? kR8 : kR4, I8 ? kCG8 : kCG4, false>),
                         dim3((unsigned)sp.NS, (unsigned)sp.S), dim3(512), 0, st, (const _Float16*)x, (const uint8_t*)W,
                         (const _Float16*)Ws, (_Float16*)y, part, counters, M, N, K, sp.S);
    return launch_status();
  }
  constexpr int C = I8 ? kC8 : kC4, P = I8 ? kP8 : kP4;
  const int NS1 = (N + 16 * C - 1) / (16 * C);
  const bool xl = (int64_t)M * K <= kXsMax;
  if (xl)
    hipLaunchKernelGGL((matvec_kernel<I8, C, kW, P, true>), dim3((unsigned)NS1), dim3(kW * 64), 0, st,
                       (const _Float16*)x, (const uint8_t*)W, (const _Float16*)Ws, (_Float16*)y, M, N, K);
  else
    hipLaunchKernelGGL((matvec_kernel<I8, C, kW, P, false>), dim3((unsigned)NS1), dim3(kW * 64), 0, st,
                       (const _Float16*)x, (const uint8_t*)W, (const _Float16*)Ws, (_Float16*)y, M, N, K);
  return launch_status();
}

// Small-M GEMM form (M > 8). Measured on MI355X (int4 / int8), K=4096:
//   M=128, N=12288: 8 columns per lane with 64-row tiles (128-column strips, 192 workgroups of 4
//     waves) 29-30 us; 4 columns with 32-row tiles and 8 waves 36-37 us; 16 columns 33-35 us.
//   M=64, N=4096: 4 columns with 16-row tiles and 16 waves 9.6-9.7 us, 8 waves 10.2-10.7 us; 8
//     columns 14-16 us.
// Wider strips cut the activation re-reads (each strip reads all of its row tile's x) and taller
// row tiles re-convert each weight fewer times, while too few workgroups leave CUs idle. So the
// 128-column strips run where they still give 192 or more workgroups and M > 32; otherwise 64-column
// strips with 16-row tiles, or 32-row tiles where 16 would give more than 3 rounds of workgroups.
// 16-row tiles take 16 waves (twice the blocks in flight per CU) where the grid is one round of at
// most 256 workgroups, and 8 waves (two workgroups per CU) beyond: at 512 workgroups 16 waves
// measured 2-3% slower, at 128-256 they measured 1-9% faster.
constexpr int kWqMaxWGs = 3 * 256, kWqMinWide = 192, kWqOneRound = 256;

template <bool I8, int C, int MT, int W, int P, bool RUNS = false>
int launch_wq_mt(int M, int N, int K, const void* x, const void* Wt, const void* Ws, void* y, hipStream_t st,
                 float* part = nullptr, unsigned* counters = nullptr, int S = 1, int QB = 0, int G = 0) {
  const dim3 grid(QB > 0 ? (unsigned)G : (unsigned)(((N + 16 * C - 1) / (16 * C)) * ((M + 16 * MT - 1) / (16 * MT))),
                  (unsigned)S);
  hipLaunchKernelGGL((gemm_wq_kernel<I8, C, MT, W, P, RUNS>), grid, dim3(W * 64), 0, st, (const _Float16*)x,
                     (const uint8_t*)Wt, (const _Float16*)Ws, (_Float16*)y, M, N, K, part, counters, S, QB);
  return launch_status();
}

// K split of the small-M GEMM (used when a workspace is given and the unsplit grid would be small):
// 128-column strips (8 columns per lane, whole 128-byte lines of int8 rows), 32-row tiles, 8 waves,
// and S splits so that about kTargetWGs workgroups run, each split at least 8 blocks. Measured at
// K=4096 against the unsplit kernel (int8 / int4): M=64, N=4096 17.1 -> 13.1 / 15.0 -> 12.1 us;
// M=128, N=4096 24.9 -> 17.4 / 22.4 -> 15.5 us; M=24, N=14336 35.3 -> 20.4 / 27.9 -> 17.2 us; M=16,
// N=4096 19.4 -> 9.7 / 17.3 -> 8.8 us. 64-column strips with 16-, 32- or 64-row tiles measured up to
// 12% faster at M <= 32, N=4096, but 25-40% slower at N=14336; 64-row tiles of 128 columns were slower
// everywhere the split applies. Workspace: the counter region, then the fp32 partials [S][M][N].
//
// Block runs (used when a workspace is given and the launch below would run more than 256 of the
// 64 x 128 tiles, filling less than 90% of their rounds of 256 workgroups, as the 384 tiles of
// M=256, N=12288 do): one workgroup per CU, each taking an equal run of QB = ceil(tiles * K/32 /
// 256) blocks of the tiles' block sequence (gemm_wq_kernel). Workspace: the counter region, then
// two fp32 partial tiles per workgroup. Measured at K=4096 (int4 / int8, whole tiles -> runs):
// M=256, N=12288 59.8 -> 55.4 / 67.8 -> 59.1 us. A single round that leaves CUs idle measured
// slower with runs (M=128, N=12288, 192 tiles: 34.4 -> 37.9 / 37.5 -> 40.6 us), so it keeps whole
// tiles.
constexpr int kWqSplitC = 8, kWqSplitMT = 2, kWqSplitW = 8;
constexpr int kWqRunC = 8, kWqRunMT = 4, kWqRunW = 4, kWqRunWGs = 256;
struct WqSplit {
  int S;         // K splits of the 32-row tiles (1: not split)
  int QB, G;     // block runs: blocks per run and workgroups (QB = 0: no runs)
  size_t bytes;  // workspace
};

// Whether the unsplit launch of launch_wq runs the 64 x 128 tiles (8 columns per lane, 4 row tiles).
bool wq_wide_tiles(int M, int N) {
  const int64_t strips4 = (N + 63) / 64, strips8 = (N + 127) / 128;
  if (M > 32 && strips8 * ((M + 63) / 64) >= kWqMinWide) return true;
  return strips4 * ((M + 15) / 16) > kWqMaxWGs && strips4 * ((M + 31) / 32) > kWqMaxWGs;
}

WqSplit wq_split_plan(int M, int N, int K) {
  WqSplit w{1, 0, 0, 0};
  if (M <= 8) return w;
  const int64_t tiles = (int64_t)((N + 16 * kWqSplitC - 1) / (16 * kWqSplitC)) *
                        ((M + 16 * kWqSplitMT - 1) / (16 * kWqSplitMT));
  int64_t S = kTargetWGs / tiles;
  if (S > kWqMaxSplits) S = kWqMaxSplits;
  if (S > K / 32 / 8) S = K / 32 / 8;
  if (S >= 2) {
    w.S = (int)S;
    w.bytes = kCounterBytes + ((size_t)S * M * N * 4 + 255) / 256 * 256;
    return w;
  }
  if (!wq_wide_tiles(M, N)) return w;
  const int64_t T = (int64_t)((N + 16 * kWqRunC - 1) / (16 * kWqRunC)) * ((M + 16 * kWqRunMT - 1) / (16 * kWqRunMT));
  const int64_t rounds = (T + kWqRunWGs - 1) / kWqRunWGs, nall = K / 32;
  if (rounds < 2 || T * 10 >= rounds * kWqRunWGs * 9 || T > (int64_t)(kCounterBytes / 4)) return w;
  const int64_t nseq = T * nall, QB = (nseq + kWqRunWGs - 1) / kWqRunWGs;
  if (QB < 8) return w;
  for (int64_t t = 0; t < T; t++)  // workgroups sharing a tile: at most kWqMaxSplits
    if (((t + 1) * nall - 1) / QB - t * nall / QB + 1 > kWqMaxSplits) return w;
  w.QB = (int)QB;
  w.G = (int)((nseq + QB - 1) / QB);
  w.bytes = kCounterBytes + (size_t)w.G * 2 * (16 * kWqRunMT) * (16 * kWqRunC) * 4;
  return w;
}

template <bool I8>
int launch_wq(int M, int N, int K, const void* x, const void* W, const void* Ws, void* y, void* ws, size_t ws_bytes,
              hipStream_t st) {
  const WqSplit sp = wq_split_plan(M, N, K);
  if ((sp.S > 1 || sp.QB > 0) && ws && ws_bytes >= sp.bytes) {
    unsigned* counters = (unsigned*)ws;
    float* part = (float*)((char*)ws + kCounterBytes);
    if (sp.QB > 0)
      return launch_wq_mt<I8, kWqRunC, kWqRunMT, kWqRunW, 2, true>(M, N, K, x, W, Ws, y, st, part, counters, 1, sp.QB, sp.G);
    return launch_wq_mt<I8, kWqSplitC, kWqSplitMT, kWqSplitW, 2>(M, N, K, x, W, Ws, y, st, part, counters, sp.S);
  }
  const int64_t strips4 = (N + 63) / 64;
  if (wq_wide_tiles(M, N)) return launch_wq_mt<I8, 8, 4, 4, 2>(M, N, K, x, W, Ws, y, st);
  if (strips4 * ((M + 15) / 16) <= kWqOneRound) return launch_wq_mt<I8, 4, 1, 16, 2>(M, N, K, x, W, Ws, y, st);
  if (strips4 * ((M + 15) / 16) <= kWqMaxWGs) return launch_wq_mt<I8, 4, 1, 8, 4>(M, N, K, x, W, Ws, y, st);
  return launch_wq_mt<I8, 4, 2, 8, 2>(M, N, K, x, W, Ws, y, st);
}

// ---- the variant that allocates nothing ---------------------------------------------------------
// The split kernel's workspace (counters, then partial sums) lives in this array instead of a
// caller buffer. Every GPU the library runs on holds its own copy until the process ends; the host
// name `scratch` is only a stand-in for it, so host code uses the address hipGetSymbolAddress gives
// for the current device and nothing else. Counters start at zero (the array is zero-initialised
// static storage, and the first call on a device also queues a clearing kernel ahead of the first
// matvec); every call leaves them at zero again.
constexpr size_t kScratchBytes = MXMATVEC_SCRATCH_BYTES;
static_assert(kScratchBytes > kCounterBytes && kScratchBytes % 256 == 0, "scratch layout");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ __launch_bounds__(256) void clear_counters_kernel(unsigned* __restrict__ c, int n) {
  const int i = (int)(blockIdx.x * 256 + threadIdx.x);
  if (i < n) c[i] = 0u;
}

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];

// Device address of this device's scratch array, set up on the first call on the device (the
// clearing kernel goes on `st`, ahead of whatever the caller queues next).
int scratch_address(hipStream_t st, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
    (void)hipGetLastError();
    return MX_ERR_ARCH;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return MX_ERR_LAUNCH;
    }
    constexpr int n = (int)(kCounterBytes / 4);
    hipLaunchKernelGGL(clear_counters_kernel, dim3((n + 255) / 256), dim3(256), 0, st, (unsigned*)p, n);
    if (hipGetLastError() != hipSuccess) return MX_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MX_OK;
}

}  // namespace

namespace mx {
size_t matvec_workspace(int M, int N, int K, bool int8) {
  return M > 8 ? wq_split_plan(M, N, K).bytes : split_plan(M, N, K, int8).bytes;
}

// mxmatvec_run with the split kernel's workspace in the static scratch array: the same kernels and
// launch shapes as a call with a large enough caller workspace, so the same results bit for bit.
int matvec_launch_noalloc(int M, int N, int K, const void* x, const void* W, bool int8, const void* Ws, void* y,
                          hipStream_t stream) {
  const size_t need = matvec_workspace(M, N, K, int8);
  if (need > kScratchBytes) return MX_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    if (int s = scratch_address(stream, &ws)) return s;
  }
  if (M > 8)
    return int8 ? launch_wq<true>(M, N, K, x, W, Ws, y, ws, need, stream)
                : launch_wq<false>(M, N, K, x, W, Ws, y, ws, need, stream);
  return int8 ? launch<true>(M, N, K, x, W, Ws, y, ws, need, stream)
              : launch<false>(M, N, K, x, W, Ws, y, ws, need, stream);
}

int matvec_launch(int M, int N, int K, const void* x, const void* W, bool int8, const void* Ws, void* y, void* ws,
                  size_t ws_bytes, hipStream_t stream) {
  if (M > 8)
    return int8 ? launch_wq<true>(M, N, K, x, W, Ws, y, ws, ws_bytes, stream)
                : launch_wq<false>(M, N, K, x, W, Ws, y, ws, ws_bytes, stream);
  return int8 ? launch<true>(M, N, K, x, W, Ws, y, ws, ws_bytes, stream)
              : launch<false>(M, N, K, x, W, Ws, y, ws, ws_bytes, stream);
}
}  // namespace mx
