// mxgemm.hip -- block-scaled (MX) GEMM and fp16 GEMM kernels for gfx950.
//
// Computes C[M,N] (fp16) = A[M,K] * B[K,N] with fp32 accumulation, where for MX operands every
// 32 consecutive K-elements of a row of A (or of a column of B) share one E8M0 scale ("TensorOps
// ... notes", sections "Scale planes" and "Kernel-phase findings"; WWDC26 session 330 summary,
// section on slicing and the quantized matmul2d). The scales are applied inside the matrix core
// by the CDNA4 scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4): no dequantised copy of any
// operand exists anywhere.
//
// Structure of one workgroup (WAVES_M x WAVES_N waves of 64 lanes; 4 or 8 waves):
//  - Output tile BM x BN; each wave owns (BM/WAVES_M) x (BN/WAVES_N) as 16x16 MFMA fragments
//    whose fp32 accumulators stay in registers for the whole K loop.
//  - K advances in stages of 128 bytes per operand row (128 E4M3 / 256 E2M1 / 64 fp16 elements).
//    Two LDS buffers alternate. The copy of stage s+1 is issued with direct global->LDS loads
//    (global_load_lds_dwordx4 / _dword: no staging registers, no LDS write instructions) before
//    the MFMAs of stage s, so it is in flight while they run; one wait + barrier ends a stage.
//    Only a K-tail stage (K not a multiple of the stage), an unaligned scale plane, or the fp16
//    right operand (which needs a transpose) take a register path instead.
//  - LDS rows are 128 bytes = 8 chunks of 16 bytes; chunk c of row r is stored at chunk
//    c ^ (r & 7). For the fragment reads (16 rows x one chunk per quarter-wave) this XOR layout
//    measured conflict-free on gfx950 (4 clocks per ds_read_b128, the 256 B/clk LDS peak), while
//    an unswizzled layout costs 4x and the variant c ^ ((r ^ (r >> 3)) & 7) 2x. A direct load
//    writes 64 lanes x 16 bytes = 8 whole rows, so each lane fetches the logical chunk that lands
//    at its physical slot.
//  - The MFMA's first operand is the B fragment and its second the A fragment, so each lane ends
//    with 4 consecutive n of one output row m and writes them with one 8-byte store.
//  - Workgroup ids are remapped so that each of the 8 XCDs (private L2 each) works on a
//    contiguous range of tiles; tiles are ordered m-fastest, so concurrently running tiles on an
//    XCD share their B panel and the A panel of the current K-window stays L2-resident.
//
// Operand lane mapping of v_mfma_scale_f32_16x16x128_f8f6f4 (measured on gfx950): lane l feeds
// row l%16; for E4M3 its 32 bytes hold K = 16q..16q+15 (bytes 0-15) and 64+16q..64+16q+15
// (bytes 16-31) with q = l/16; for E2M1 its 16 bytes hold K = 32q..32q+31, the even K in the low
// nibble. The scale byte given by lane group b (selected by op_sel) applies to K-block b of the
// 128-wide MFMA step. The fp16 MFMA (16x16x32) takes K = 8q..8q+7 per lane.
#include "common.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;

enum Kind { KIND_E4M3 = 0, KIND_E2M1 = 1, KIND_F16 = 2 };

constexpr int kRowBytes = 128;  // bytes of one operand row per pipeline stage

MX_DEV int swz(int row) { return row & 7; }
MX_DEV int lds_off(int row, int chunk) { return row * kRowBytes + ((chunk ^ swz(row)) << 4); }

template <int KIND, int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NWAVES = WAVES_M * WAVES_N, THREADS = 64 * NWAVES;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int KSTEP = KIND == KIND_E4M3 ? 128 : (KIND == KIND_E2M1 ? 256 : 64);
  static constexpr int NSB = KSTEP / 32;  // E8M0 bytes per row per stage
  static constexpr int TILE_BYTES = (BM + BN) * kRowBytes;
  static constexpr int SCALE_DW = KIND == KIND_F16 ? 0 : (BM + BN) * NSB / 4;  // scale dwords per stage
  static constexpr int STAGE_BYTES = TILE_BYTES + 4 * SCALE_DW;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  // direct loads: one wave instruction moves 8 rows (16 B per lane) or 64 scale dwords; the
  // instructions of a stage are dealt round-robin to the waves
  static constexpr int ROW_INSTR = (BM + (KIND == KIND_F16 ? 0 : BN)) / 8;
  static constexpr int S_INSTR = (SCALE_DW + 63) / 64;
  // register path (tail stage / fp16 right operand)
  static constexpr int A_CHUNKS = (BM * 8 + THREADS - 1) / THREADS;
  static constexpr int B_CHUNKS = KIND == KIND_F16 ? 0 : (BN * 8 + THREADS - 1) / THREADS;
  static constexpr int B_MICRO = KIND == KIND_F16 ? (BN + THREADS - 1) / THREADS : 0;  // 8x8 fp16 blocks
  static_assert(BM % 32 == 0 && BN % 32 == 0 && WM % 16 == 0 && WN % 16 == 0, "tile");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

struct Args {
  const uint8_t* A;
  const uint8_t* SA;
  const uint8_t* B;
  const uint8_t* SB;
  _Float16* C;
  int M, N, K;
  int tiles_m, tiles_n;
  int64_t a_row_bytes;  // bytes of one row of A (and of B for MX kinds)
  int nblk;             // K / 32
  int nstages;
  int relu;             // epilogue: C = max(C, 0) (IEEE maxNum: NaN gives 0)
};

MX_DEV void g2l(const void* g, char* lds_wave_base, int size) {
  if (size == 16)
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)g, (lds_ptr_t)lds_wave_base, 16, 0, 0);
  else
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)g, (lds_ptr_t)lds_wave_base, 4, 0, 0);
}

// Buffer resources (scalar registers) over the tile's rows of A, B and their scale planes. Direct
// copies address them with a loop-invariant 32-bit per-lane offset (VGPR) plus a wave-uniform
// offset (SGPR), which keeps per-instruction addresses out of the vector register file.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;  // raw (untyped) buffer, 32-bit data format, no swizzle

MX_DEV rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcFlags);
}

MX_DEV void b2l(rsrc_t r, char* lds_wave_base, uint32_t voff, uint32_t soff, int size) {
  if (size == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_wave_base, 16, voff, soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_wave_base, 4, voff, soff, 0, 0);
}

struct TileSrc {
  rsrc_t a, b, sa, sb;   // rows [m0, m0+rows_a) of A/SA and [n0, n0+rows_b) of B/SB
  int rows_a, rows_b;
};

template <class CF>
MX_DEV TileSrc tile_src(const Args& p, int m0, int n0) {
  TileSrc t;
  t.rows_a = min(CF::BM, p.M - m0);
  t.rows_b = min(CF::BN, p.N - n0);
  t.a = make_rsrc(p.A + (int64_t)m0 * p.a_row_bytes, (uint32_t)(t.rows_a * p.a_row_bytes));
  t.b = make_rsrc(p.B + (int64_t)n0 * p.a_row_bytes, (uint32_t)(t.rows_b * p.a_row_bytes));
  t.sa = make_rsrc(p.SA + (int64_t)m0 * p.nblk, (uint32_t)(t.rows_a * p.nblk));
  t.sb = make_rsrc(p.SB + (int64_t)n0 * p.nblk, (uint32_t)(t.rows_b * p.nblk));
  return t;
}

// Direct copy of the code rows of stage s (A, and B for MX kinds) into one LDS stage buffer.
// Lane l of an instruction fills tile row r0 + l/8, physical chunk l%8; with the (row & 7)
// swizzle its byte offset inside the 8-row group, (l/8)*row_bytes + ((l%8) ^ (l/8))*16, is the
// same for every instruction. Groups that reach past the last row clamp each lane's row instead.
template <class CF, int KIND, int NW = CF::NWAVES>
MX_DEV void issue_direct_rows(const Args& p, const TileSrc& t, char* buf, int s, int wave, int lane) {
  const uint32_t kbyte0 = (uint32_t)(s * kRowBytes), rb = (uint32_t)p.a_row_bytes;
  const int rsub = lane >> 3, pch = lane & 7;
  const uint32_t chunk_off = (uint32_t)((pch ^ rsub) << 4), lane_off = (uint32_t)rsub * rb + chunk_off;
#pragma unroll
  for (int i0 = 0; i0 < CF::ROW_INSTR; i0 += NW) {
    const int i = i0 + wave;
    if (CF::ROW_INSTR % NW == 0 || i < CF::ROW_INSTR) {
      const int r0 = i * 8;  // tile row: A rows first, then B rows
      const bool isA = r0 < CF::BM;
      const int rloc = isA ? r0 : r0 - CF::BM;
      const int rows = isA ? t.rows_a : t.rows_b;
      const rsrc_t r = isA ? t.a : t.b;
      if (rloc + 8 <= rows) {
        b2l(r, buf + r0 * kRowBytes, lane_off, (uint32_t)rloc * rb + kbyte0, 16);
      } else {
        const int cr = min(rloc + rsub, rows - 1);
        b2l(r, buf + r0 * kRowBytes, (uint32_t)cr * rb + kbyte0 + chunk_off, 0u, 16);
      }
    }
  }
}

// Direct copy of the stage's scale dwords (A rows then B rows, NSB bytes each); needs K/32 % 4 == 0.
// Instruction i covers scale dwords 64i..64i+63, i.e. 64 / (NSB/4) rows.
template <class CF, int NW = CF::NWAVES>
MX_DEV void issue_direct_scales(const Args& p, const TileSrc& t, char* buf, int s, int wave, int lane) {
  constexpr int per_row = CF::NSB / 4, rows_per_instr = 64 / per_row;
  static_assert(CF::BM % rows_per_instr == 0, "scale instructions must not straddle A and B rows");
  const int lrow = lane / per_row, ldw = lane % per_row;
  const uint32_t nb = (uint32_t)p.nblk, sbyte0 = (uint32_t)(s * CF::NSB);
  const uint32_t lane_off = (uint32_t)lrow * nb + 4 * ldw;
#pragma unroll
  for (int i = wave; i < CF::S_INSTR; i += NW) {
    const int did = i * 64 + lane;
    if (did < CF::SCALE_DW) {
      const int r0 = i * rows_per_instr;
      const bool isA = r0 < CF::BM;
      const int rloc = isA ? r0 : r0 - CF::BM;
      const int rows = isA ? t.rows_a : t.rows_b;
      const rsrc_t r = isA ? t.sa : t.sb;
      if (rloc + rows_per_instr <= rows) {
        b2l(r, buf + CF::TILE_BYTES + i * 256, lane_off, (uint32_t)rloc * nb + sbyte0, 4);
      } else {
        const int cr = min(rloc + lrow, rows - 1);
        b2l(r, buf + CF::TILE_BYTES + i * 256, (uint32_t)cr * nb + sbyte0 + 4 * ldw, 0u, 4);
      }
    }
  }
}

// Register path for one stage: zero-filled codes past K, scale 127 (= 1.0) for blocks past K.
template <class CF, int KIND, int NTHR = CF::THREADS>
MX_DEV void copy_stage_regs(const Args& p, char* buf, int m0, int n0, int s, int tid, bool rows, bool scales) {
  const int64_t kbyte0 = (int64_t)s * kRowBytes;
  constexpr int A_CH = (CF::BM * 8 + NTHR - 1) / NTHR;
  constexpr int B_CH = KIND == KIND_F16 ? 0 : (CF::BN * 8 + NTHR - 1) / NTHR;
  if (rows) {
#pragma unroll
    for (int i = 0; i < A_CH; i++) {
      const int cid = tid + NTHR * i, row = cid >> 3, cc = cid & 7;
      if (cid >= CF::BM * 8) break;
      const int gr = min(m0 + row, p.M - 1);
      const int64_t kb = kbyte0 + cc * 16;
      const v4i v = kb < p.a_row_bytes ? *reinterpret_cast<const v4i*>(p.A + (int64_t)gr * p.a_row_bytes + kb)
                                       : v4i{0, 0, 0, 0};
      *reinterpret_cast<v4i*>(buf + lds_off(row, cc)) = v;
    }
#pragma unroll
    for (int i = 0; i < B_CH; i++) {
      const int cid = tid + NTHR * i, row = cid >> 3, cc = cid & 7;
      if (cid >= CF::BN * 8) break;
      const int gr = min(n0 + row, p.N - 1);
      const int64_t kb = kbyte0 + cc * 16;
      const v4i v = kb < p.a_row_bytes ? *reinterpret_cast<const v4i*>(p.B + (int64_t)gr * p.a_row_bytes + kb)
                                       : v4i{0, 0, 0, 0};
      *reinterpret_cast<v4i*>(buf + lds_off(CF::BM + row, cc)) = v;
    }
  }
  if constexpr (KIND != KIND_F16) {
    if (scales) {
      constexpr int per_row = CF::NSB / 4;
      uint32_t* sl = reinterpret_cast<uint32_t*>(buf + CF::TILE_BYTES);
      for (int did = tid; did < CF::SCALE_DW; did += NTHR) {
        const int row = did / per_row, dw = did % per_row;
        const bool isA = row < CF::BM;
        const int gr = isA ? min(m0 + row, p.M - 1) : min(n0 + row - CF::BM, p.N - 1);
        const uint8_t* srow = (isA ? p.SA : p.SB) + (int64_t)gr * p.nblk;
        const int b = s * CF::NSB + 4 * dw;
        uint32_t v = 0u;
#pragma unroll
        for (int j = 0; j < 4; j++) v |= (uint32_t)(b + j < p.nblk ? srow[b + j] : 127u) << (8 * j);
        sl[did] = v;
      }
    }
  }
}

// fp16 right operand B[K][N] (row-major): each thread reads an 8 (k) x 8 (n) block with eight
// 16-byte row loads and stores it transposed (n-major, 8 k per chunk) after the stage's MFMAs.
template <class CF>
struct BTrans {
  v4i r[CF::B_MICRO > 0 ? CF::B_MICRO * 8 : 1];
};

template <class CF>
MX_DEV void load_btrans(BTrans<CF>& bt, const Args& p, int n0, int s, int tid) {
#pragma unroll
  for (int u = 0; u < CF::B_MICRO; u++) {
    const int mb = tid + CF::THREADS * u;
    constexpr int nchunks = CF::BN / 8;
    const int nc = mb % nchunks, kg = mb / nchunks;
    const int n = n0 + nc * 8;
#pragma unroll
    for (int r = 0; r < 8; r++) {
      const int k = s * 64 + kg * 8 + r;
      const bool ok = mb < CF::BN && k < p.K && n < p.N;
      bt.r[u * 8 + r] = ok ? *reinterpret_cast<const v4i*>(p.B + ((int64_t)k * p.N + n) * 2) : v4i{0, 0, 0, 0};
    }
  }
}

template <class CF>
MX_DEV void store_btrans(const BTrans<CF>& bt, char* buf, int tid) {
#pragma unroll
  for (int u = 0; u < CF::B_MICRO; u++) {
    const int mb = tid + CF::THREADS * u;
    if (mb >= CF::BN) break;
    constexpr int nchunks = CF::BN / 8;
    const int nc = mb % nchunks, kg = mb / nchunks;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int p2 = j >> 1;
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      v4i o;
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const uint32_t lo = (uint32_t)bt.r[u * 8 + 2 * q][p2], hi = (uint32_t)bt.r[u * 8 + 2 * q + 1][p2];
        o[q] = (int)__builtin_amdgcn_perm(hi, lo, sel);
      }
      *reinterpret_cast<v4i*>(buf + lds_off(CF::BM + nc * 8 + j, kg)) = o;
    }
  }
}

// Workgroup barrier without the release/acquire fences of __syncthreads(): those fences make the
// compiler wait for every outstanding direct global->LDS load (vmcnt(0)) at each barrier, which
// would serialise the next stage's copy into the current one. The memory clobber keeps the
// compiler from moving memory operations across it; the waits the protocol needs are explicit:
// wait_lds() before a barrier that releases an LDS buffer for overwriting, wait_vm() before a
// barrier that publishes a direct copy.
MX_DEV void raw_barrier() { asm volatile("s_barrier" ::: "memory"); }
MX_DEV void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0) only
MX_DEV void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0) only

MX_DEV v4i lds_read16(const char* lds, int row, int chunk) {
  return *reinterpret_cast<const v4i*>(lds + lds_off(row, chunk));
}

MX_DEV v8i widen(v4i x) { return __builtin_shufflevector(x, x, 0, 1, 2, 3, -1, -1, -1, -1); }
MX_DEV v8i cat(v4i a, v4i b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }

// MFMAs of one stage from LDS buffer `buf`.
template <class CF, int KIND>
MX_DEV void compute_stage(const char* buf, v4f (&acc)[CF::FN][CF::FM], int wm, int wn, int r16, int q) {
  const uint8_t* sc = reinterpret_cast<const uint8_t*>(buf + CF::TILE_BYTES);
  if constexpr (KIND == KIND_E4M3) {
    v8i af[CF::FM];
    int sa[CF::FM];
#pragma unroll
    for (int j = 0; j < CF::FM; j++) {
      const int row = wm * CF::WM + 16 * j + r16;
      af[j] = cat(lds_read16(buf, row, q), lds_read16(buf, row, 4 + q));
      sa[j] = sc[row * CF::NSB + q];
    }
#pragma unroll
    for (int i = 0; i < CF::FN; i++) {
      const int row = CF::BM + wn * CF::WN + 16 * i + r16;
      const v8i bf = cat(lds_read16(buf, row, q), lds_read16(buf, row, 4 + q));
      const int sb = sc[row * CF::NSB + q];
#pragma unroll
      for (int j = 0; j < CF::FM; j++)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[j], acc[i][j], 0, 0, 0, sb, 0, sa[j]);
    }
  } else if constexpr (KIND == KIND_E2M1) {
    // scale bytes: byte h of each lane's scale register is the block of K-half h
    int sa[CF::FM], sb[CF::FN];
#pragma unroll
    for (int j = 0; j < CF::FM; j++) {
      const int row = wm * CF::WM + 16 * j + r16;
      sa[j] = sc[row * CF::NSB + q] | (sc[row * CF::NSB + 4 + q] << 8);
    }
#pragma unroll
    for (int i = 0; i < CF::FN; i++) {
      const int row = CF::BM + wn * CF::WN + 16 * i + r16;
      sb[i] = sc[row * CF::NSB + q] | (sc[row * CF::NSB + 4 + q] << 8);
    }
#pragma unroll
    for (int h = 0; h < 2; h++) {
      v8i af[CF::FM];
#pragma unroll
      for (int j = 0; j < CF::FM; j++) af[j] = widen(lds_read16(buf, wm * CF::WM + 16 * j + r16, 4 * h + q));
#pragma unroll
      for (int i = 0; i < CF::FN; i++) {
        const v8i bf = widen(lds_read16(buf, CF::BM + wn * CF::WN + 16 * i + r16, 4 * h + q));
#pragma unroll
        for (int j = 0; j < CF::FM; j++) {
          if (h == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[j], acc[i][j], 4, 4, 0, sb[i], 0, sa[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[j], acc[i][j], 4, 4, 1, sb[i], 1, sa[j]);
        }
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; h++) {
      v8h af[CF::FM];
#pragma unroll
      for (int j = 0; j < CF::FM; j++)
        af[j] = __builtin_bit_cast(v8h, lds_read16(buf, wm * CF::WM + 16 * j + r16, 4 * h + q));
#pragma unroll
      for (int i = 0; i < CF::FN; i++) {
        const v8h bf = __builtin_bit_cast(v8h, lds_read16(buf, CF::BM + wn * CF::WN + 16 * i + r16, 4 * h + q));
#pragma unroll
        for (int j = 0; j < CF::FM; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf, af[j], acc[i][j], 0, 0, 0);
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// Epilogue shared by the 16x16-MFMA kernels: fp32 -> fp16 (nearest even). acc[i][j] holds, in lane
// l, C[mb + 16j + l%16][nb + 16i + 4(l/16) + v] for v = 0..3: 8 bytes of a row, so stores straight
// from registers would write every 128-byte line of C in pieces from several instructions. The
// wave instead writes 16 rows at a time into its own LDS scratch (row pitch 2*WN + 16 bytes: the
// 8-byte writes of 16 rows x 2 column groups land on distinct banks) and stores them back as
// 16-byte pieces, consecutive lanes along a row.
template <class CF>
constexpr int C_PITCH = 2 * CF::WN + 16;

template <class CF>
MX_DEV void store_c(const Args& p, v4f (&acc)[CF::FN][CF::FM], char* ws, int mb, int nb, int lane) {
  static_assert(CF::NWAVES * 16 * C_PITCH<CF> <= CF::LDS_BYTES, "epilogue scratch");
  typedef _Float16 v8h __attribute__((ext_vector_type(8)));
  constexpr int LPR = CF::WN / 8;  // 16-byte pieces per row
  constexpr int PIECES = 16 * LPR;
  const int r16 = lane & 15, q = lane >> 4;
  const bool rows16 = (p.N & 7) == 0, rows8 = (p.N & 3) == 0;  // row starts 16- / 8-byte aligned
  if (p.relu) {  // (one uniform branch, not a select per element)
#pragma unroll
    for (int i = 0; i < CF::FN; i++)
#pragma unroll
      for (int j = 0; j < CF::FM; j++)
#pragma unroll
        for (int v = 0; v < 4; v++) acc[i][j][v] = fmaxf(acc[i][j][v], 0.0f);
  }
#pragma unroll
  for (int j = 0; j < CF::FM; j++) {
#pragma unroll
    for (int i = 0; i < CF::FN; i++) {
      const v4f a = acc[i][j];
      *reinterpret_cast<v4h*>(ws + r16 * C_PITCH<CF> + (16 * i + 4 * q) * 2) =
          v4h{(_Float16)a[0], (_Float16)a[1], (_Float16)a[2], (_Float16)a[3]};
    }
#pragma unroll
    for (int s0 = 0; s0 < PIECES; s0 += 64) {
      const int piece = s0 + lane;
      if (PIECES % 64 != 0 && piece >= PIECES) continue;
      const int lr = piece / LPR, c = piece % LPR;
      const v8h v = *reinterpret_cast<const v8h*>(ws + lr * C_PITCH<CF> + 16 * c);
      const int m = mb + 16 * j + lr, n = nb + 8 * c;
      if (m >= p.M) continue;
      _Float16* dst = p.C + (int64_t)m * p.N + n;
      // non-temporal stores: C streams out without displacing operand panels from the caches
      if (rows16 && n + 8 <= p.N) {
        __builtin_nontemporal_store(v, reinterpret_cast<v8h*>(dst));
      } else if (rows8 && n + 8 <= p.N) {
        __builtin_nontemporal_store(__builtin_shufflevector(v, v, 0, 1, 2, 3), reinterpret_cast<v4h*>(dst));
        __builtin_nontemporal_store(__builtin_shufflevector(v, v, 4, 5, 6, 7), reinterpret_cast<v4h*>(dst + 4));
      } else {
#pragma unroll
        for (int e = 0; e < 8; e++)
          if (n + e < p.N) dst[e] = v[e];
      }
    }
  }
}

template <class CF, int KIND>
__global__ __launch_bounds__(CF::THREADS, 1) void gemm_kernel(Args p) {
  __shared__ __attribute__((aligned(16))) char lds[CF::LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) index
  const int wm = wave % CF::WAVES_M, wn = wave / CF::WAVES_M;
  const int r16 = lane & 15, q = lane >> 4;

  // XCD-aware tile order (see file comment).
  int bid = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);
  const int tm = bid % p.tiles_m, tn = bid / p.tiles_m;
  const int m0 = tm * CF::BM, n0 = tn * CF::BN;
  const bool aligned_scales = (p.nblk & 3) == 0;

  v4f acc[CF::FN][CF::FM];
#pragma unroll
  for (int i = 0; i < CF::FN; i++)
#pragma unroll
    for (int j = 0; j < CF::FM; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Start the copy of stage s into buffer b. Returns after queueing direct loads (full stages)
  // or after finishing register copies (tail stage, unaligned scales).
  const TileSrc tsrc = tile_src<CF>(p, m0, n0);
  auto start_stage = [&](int s, char* buf) {
    const bool full = (int64_t)(s + 1) * kRowBytes <= p.a_row_bytes;
    if (full) issue_direct_rows<CF, KIND>(p, tsrc, buf, s, wave, lane);
    if constexpr (KIND != KIND_F16) {
      if (full && aligned_scales) issue_direct_scales<CF>(p, tsrc, buf, s, wave, lane);
      if (!full || !aligned_scales) copy_stage_regs<CF, KIND>(p, buf, m0, n0, s, tid, !full, true);
    } else {
      if (!full) copy_stage_regs<CF, KIND>(p, buf, m0, n0, s, tid, true, false);
    }
  };

  BTrans<CF> bt;
  start_stage(0, lds);
  if constexpr (KIND == KIND_F16) {
    load_btrans<CF>(bt, p, n0, 0, tid);
    store_btrans<CF>(bt, lds, tid);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int s = 0; s < p.nstages; s++) {
    char* cur = lds + (s & 1) * CF::STAGE_BYTES;
    char* nxt = lds + ((s + 1) & 1) * CF::STAGE_BYTES;
    const bool more = s + 1 < p.nstages;
    if (more) {
      start_stage(s + 1, nxt);
      if constexpr (KIND == KIND_F16) load_btrans<CF>(bt, p, n0, s + 1, tid);
    }
    compute_stage<CF, KIND>(cur, acc, wm, wn, r16, q);
    if constexpr (KIND == KIND_F16) {
      __builtin_amdgcn_sched_barrier(0);
      if (more) store_btrans<CF>(bt, nxt, tid);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies (direct and register) have landed in LDS
    raw_barrier();                  // ... and every other wave's
  }

  // Epilogue: every wave is past the last stage's barrier, so the stage buffers are free.
  store_c<CF>(p, acc, lds + wave * 16 * C_PITCH<CF>, m0 + wm * CF::WM, n0 + wn * CF::WN, lane);
}


// ------------------------------------------------------------------------------------------------
// Ping-pong variant for the MX formats (8 waves, 4 x 2, two per SIMD).
//
// Waves 0-3 (group 0, left half of the tile's N) and waves 4-7 (group 1, right half) run half a
// stage apart. Each wave alternates a load phase (LDS -> registers: its A/B fragments and scale
// bytes of one stage; plus its 1/8 share of a direct global->LDS stage copy) and a compute phase
// (all MFMAs of the stage, from registers only). While one wave of a SIMD computes, its partner
// loads, so the matrix core always has an instruction stream, and the (blocking) issue of the
// copy loads never sits inside an MFMA stream. Stage t lives in buffer t&1:
//   phase 2t   : group 0 queues its share of stage t+1 (buffer (t+1)&1), reads stage t
//                group 1 computes stage t-1
//   phase 2t+1 : group 0 computes stage t
//                group 1 reads stage t, then queues its share of stage t+2 into buffer t&1
// A copy into a buffer starts only after both groups have read the stage it replaces; each group
// waits for its own copies at the end of its compute phase, before the stage is first read.
// Stages 0 and 1 are copied by all waves before the loop. Workgroup barriers separate phases and
// both groups execute the same number of them.
// ------------------------------------------------------------------------------------------------
template <class CF, int KIND>
struct Frags {
  // E4M3: one 32-byte fragment per 16 rows; E2M1: two 16-byte halves (K-halves of the stage)
  v8i a8[KIND == KIND_E4M3 ? CF::FM : 1], b8[KIND == KIND_E4M3 ? CF::FN : 1];
  v4i a4[KIND == KIND_E2M1 ? CF::FM : 1][2], b4[KIND == KIND_E2M1 ? CF::FN : 1][2];
  int sa[CF::FM], sb[CF::FN];
};

template <class CF, int KIND>
MX_DEV void load_frags(Frags<CF, KIND>& f, const char* buf, int wm, int wn, int r16, int q) {
  const uint8_t* sc = reinterpret_cast<const uint8_t*>(buf + CF::TILE_BYTES);
#pragma unroll
  for (int j = 0; j < CF::FM; j++) {
    const int row = wm * CF::WM + 16 * j + r16;
    if constexpr (KIND == KIND_E4M3) {
      f.a8[j] = cat(lds_read16(buf, row, q), lds_read16(buf, row, 4 + q));
      f.sa[j] = sc[row * CF::NSB + q];
    } else {
      f.a4[j][0] = lds_read16(buf, row, q);
      f.a4[j][1] = lds_read16(buf, row, 4 + q);
      f.sa[j] = sc[row * CF::NSB + q] | (sc[row * CF::NSB + 4 + q] << 8);
    }
  }
#pragma unroll
  for (int i = 0; i < CF::FN; i++) {
    const int row = CF::BM + wn * CF::WN + 16 * i + r16;
    if constexpr (KIND == KIND_E4M3) {
      f.b8[i] = cat(lds_read16(buf, row, q), lds_read16(buf, row, 4 + q));
      f.sb[i] = sc[row * CF::NSB + q];
    } else {
      f.b4[i][0] = lds_read16(buf, row, q);
      f.b4[i][1] = lds_read16(buf, row, 4 + q);
      f.sb[i] = sc[row * CF::NSB + q] | (sc[row * CF::NSB + 4 + q] << 8);
    }
  }
}

// Route every fragment register through an empty volatile asm, ordered after the preceding
// barrier, so the MFMAs that consume them cannot be scheduled before it.
template <class CF, int KIND>
MX_DEV void pin_frags(Frags<CF, KIND>& f) {
#pragma unroll
  for (int j = 0; j < CF::FM; j++) {
    if constexpr (KIND == KIND_E4M3) asm volatile("" : "+v"(f.a8[j]));
    else asm volatile("" : "+v"(f.a4[j][0]), "+v"(f.a4[j][1]));
    asm volatile("" : "+v"(f.sa[j]));
  }
#pragma unroll
  for (int i = 0; i < CF::FN; i++) {
    if constexpr (KIND == KIND_E4M3) asm volatile("" : "+v"(f.b8[i]));
    else asm volatile("" : "+v"(f.b4[i][0]), "+v"(f.b4[i][1]));
    asm volatile("" : "+v"(f.sb[i]));
  }
}

template <class CF, int KIND>
MX_DEV void mfma_frags(const Frags<CF, KIND>& f, v4f (&acc)[CF::FN][CF::FM]) {
  if constexpr (KIND == KIND_E4M3) {
#pragma unroll
    for (int i = 0; i < CF::FN; i++)
#pragma unroll
      for (int j = 0; j < CF::FM; j++)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.b8[i], f.a8[j], acc[i][j], 0, 0, 0, f.sb[i], 0, f.sa[j]);
  } else {
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
      for (int i = 0; i < CF::FN; i++)
#pragma unroll
        for (int j = 0; j < CF::FM; j++) {
          if (h == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(widen(f.b4[i][0]), widen(f.a4[j][0]), acc[i][j], 4,
                                                                         4, 0, f.sb[i], 0, f.sa[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(widen(f.b4[i][1]), widen(f.a4[j][1]), acc[i][j], 4,
                                                                         4, 1, f.sb[i], 1, f.sa[j]);
        }
  }
}

template <class CF, int KIND>
MX_DEV void pin_acc(v4f (&acc)[CF::FN][CF::FM]) {
#pragma unroll
  for (int i = 0; i < CF::FN; i++)
#pragma unroll
    for (int j = 0; j < CF::FM; j++) asm volatile("" : "+v"(acc[i][j]));
}

template <class CF, int KIND>
__global__ __launch_bounds__(CF::THREADS, 1) void gemm_pp_kernel(Args p) {
  static_assert(CF::WAVES_M == 4 && CF::WAVES_N == 2 && KIND != KIND_F16, "ping-pong layout");
  __shared__ __attribute__((aligned(16))) char lds[CF::LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) index
  const int wm = wave % CF::WAVES_M, wn = wave / CF::WAVES_M;  // group = wn
  const int r16 = lane & 15, q = lane >> 4;
  const int gw = wave & 3;                                     // wave index inside its group

  int bid = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);
  const int tm = bid % p.tiles_m, tn = bid / p.tiles_m;
  const int m0 = tm * CF::BM, n0 = tn * CF::BN;

  v4f acc[CF::FN][CF::FM];
#pragma unroll
  for (int i = 0; i < CF::FN; i++)
#pragma unroll
    for (int j = 0; j < CF::FM; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // The host uses this kernel only when every stage is full (K a multiple of the stage) and the
  // scale rows are dword aligned (K/32 % 4 == 0). Prologue: all 8 waves copy stages 0 and 1.
  const TileSrc tsrc = tile_src<CF>(p, m0, n0);
  issue_direct_rows<CF, KIND, 8>(p, tsrc, lds, 0, wave, lane);
  issue_direct_scales<CF, 8>(p, tsrc, lds, 0, wave, lane);
  if (p.nstages > 1) {
    issue_direct_rows<CF, KIND, 8>(p, tsrc, lds + CF::STAGE_BYTES, 1, wave, lane);
    issue_direct_scales<CF, 8>(p, tsrc, lds + CF::STAGE_BYTES, 1, wave, lane);
  }
  __builtin_amdgcn_s_waitcnt(0);
  raw_barrier();

  Frags<CF, KIND> f;
  if (wn == 0) {
    for (int t = 0; t < p.nstages; t++) {
      char* cur = lds + (t & 1) * CF::STAGE_BYTES;
      if (t >= 1 && t + 1 < p.nstages) {  // phase 2t: this wave's share of stage t+1
        char* nxt = lds + ((t + 1) & 1) * CF::STAGE_BYTES;
        issue_direct_rows<CF, KIND, 8>(p, tsrc, nxt, t + 1, wave, lane);
        issue_direct_scales<CF, 8>(p, tsrc, nxt, t + 1, wave, lane);
      }
      load_frags<CF, KIND>(f, cur, wm, wn, r16, q);
      wait_lds();
      raw_barrier();
      pin_frags<CF, KIND>(f);
      mfma_frags<CF, KIND>(f, acc);  // phase 2t+1
      pin_acc<CF, KIND>(acc);
      wait_vm();                     // the share of stage t+1 queued in phase 2t has landed
      raw_barrier();
    }
    raw_barrier();
  } else {
    raw_barrier();  // phase 0
    for (int t = 0; t < p.nstages; t++) {
      char* cur = lds + (t & 1) * CF::STAGE_BYTES;
      load_frags<CF, KIND>(f, cur, wm, wn, r16, q);  // phase 2t+1
      wait_lds();
      if (t + 2 < p.nstages) {  // this wave's share of stage t+2 into the buffer just read
        issue_direct_rows<CF, KIND, 8>(p, tsrc, cur, t + 2, wave, lane);
        issue_direct_scales<CF, 8>(p, tsrc, cur, t + 2, wave, lane);
      }
      raw_barrier();
      pin_frags<CF, KIND>(f);
      mfma_frags<CF, KIND>(f, acc);  // phase 2t+2
      pin_acc<CF, KIND>(acc);
      wait_vm();                     // the share of stage t+2 queued in phase 2t+1 has landed
      raw_barrier();
    }
  }

  // Epilogue: every wave is past its last barrier, so the stage buffers are free.
  store_c<CF>(p, acc, lds + wave * 16 * C_PITCH<CF>, m0 + wm * CF::WM, n0 + wn * CF::WN, lane);
}

template <int KIND, int BM, int BN>
int launch_pp(const Args& a0, hipStream_t stream) {
  if constexpr (KIND == KIND_F16) {
    return MX_ERR_FORMAT;
  } else {
    using CF = Cfg<KIND, BM, BN, 4, 2>;
    if (a0.a_row_bytes % kRowBytes != 0 || (a0.nblk & 3) != 0) return launch<KIND, BM, BN, 4, 2>(a0, stream);
    Args a = a0;
    a.tiles_m = (a.M + BM - 1) / BM;
    a.tiles_n = (a.N + BN - 1) / BN;
    a.nstages = (int)((a.a_row_bytes + kRowBytes - 1) / kRowBytes);
    const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
    if (tiles > 0x7FFFFFFF) return MX_ERR_SHAPE;
    hipLaunchKernelGGL((gemm_pp_kernel<CF, KIND>), dim3((unsigned)tiles), dim3(CF::THREADS), 0, stream, a);
    return mx::launch_status();
  }
}

template <int KIND, int BM, int BN, int WGM, int WGN>
int launch(const Args& a0, hipStream_t stream) {
  using CF = Cfg<KIND, BM, BN, WGM, WGN>;
  Args a = a0;
  a.tiles_m = (a.M + BM - 1) / BM;
  a.tiles_n = (a.N + BN - 1) / BN;
  a.nstages = (int)((a.a_row_bytes + kRowBytes - 1) / kRowBytes);
  const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
  if (tiles > 0x7FFFFFFF) return MX_ERR_SHAPE;
  hipLaunchKernelGGL((gemm_kernel<CF, KIND>), dim3((unsigned)tiles), dim3(CF::THREADS), 0, stream, a);
  return mx::launch_status();
}

}  // namespace

namespace mx {

int gemm_ring_launch(int kind, int bn, int fca, int fcb, const void* A, const void* SA, const void* B,
                     const void* SB, void* C, int M, int N, int K, bool relu, hipStream_t stream);
int gemm_pp_ring_launch(int kind, int fca, int fcb, const void* A, const void* SA, const void* B, const void* SB,
                        void* C, int M, int N, int K, bool relu, bool qa, hipStream_t stream);

// Tile configurations, indexed by the plan. Returns MX_ERR_FORMAT for an unknown id.
// qa: A is binary16 and quantised to E4M3 on load (kind E4M3 on tile 11 only; checked by the caller).
int gemm_launch(int kind, int tile_id, const void* A, const void* SA, const void* B, const void* SB, void* C, int M,
                int N, int K, bool relu, bool qa, hipStream_t stream) {
  if (qa) return gemm_pp_ring_launch(0, 0, 0, A, SA, B, SB, C, M, N, K, relu, true, stream);
  // The other pairs: 3: E4M3 A x E2M1 B, 4: E2M1 A x E4M3 B (the ring, 256x256 or 256x224 tiles);
  // with E5M2: 5: E5M2 x E5M2, 6: E4M3 x E5M2, 7: E5M2 x E4M3, 8: E5M2 x E2M1, 9: E2M1 x E5M2;
  // FP6: 10: E2M3 x E2M3, 11: E3M2 x E3M2, 12: E2M3 x E3M2, 13: E3M2 x E2M3. All of them run on the
  // ping-pong ring on tile 11 where K % 1024 == 0 and N % 4 == 0; otherwise on the 256x256 ring.
  if (kind >= 5 && kind <= 7 && tile_id == 11 && K % 1024 == 0 && N % 4 == 0) {
    static const int pfa[3] = {1, 0, 1}, pfb[3] = {1, 1, 0};
    return gemm_pp_ring_launch(0, pfa[kind - 5], pfb[kind - 5], A, SA, B, SB, C, M, N, K, relu, false, stream);
  }
  if (kind >= 10 && kind <= 13 && tile_id == 11 && K % 1024 == 0 && N % 4 == 0) {
    static const int pfa[4] = {2, 3, 2, 3}, pfb[4] = {2, 3, 3, 2};
    return gemm_pp_ring_launch(5, pfa[kind - 10], pfb[kind - 10], A, SA, B, SB, C, M, N, K, relu, false, stream);
  }
  if ((kind == 3 || kind == 8) && tile_id == 11 && K % 1024 == 0 && N % 4 == 0)  // byte A x E2M1 B
    return gemm_pp_ring_launch(2, kind == 3 ? 0 : 1, 4, A, SA, B, SB, C, M, N, K, relu, false, stream);
  if ((kind == 4 || kind == 9) && tile_id == 11 && K % 1024 == 0 && N % 4 == 0)  // E2M1 A x byte B
    return gemm_pp_ring_launch(3, 4, kind == 4 ? 0 : 1, A, SA, B, SB, C, M, N, K, relu, false, stream);
  if (kind == 3 || kind == 4)
    return gemm_ring_launch(kind - 1, tile_id == 9 ? 224 : 256, 0, 0, A, SA, B, SB, C, M, N, K, relu, stream);
  if (kind >= 5 && kind <= 13) {
    static const int rk[9] = {0, 0, 0, 2, 3, 5, 5, 5, 5};
    static const int fa[9] = {1, 0, 1, 1, 0, 2, 3, 2, 3}, fb[9] = {1, 1, 0, 0, 1, 2, 3, 3, 2};
    return gemm_ring_launch(rk[kind - 5], 256, fa[kind - 5], fb[kind - 5], A, SA, B, SB, C, M, N, K, relu, stream);
  }
  Args a{};
  a.A = (const uint8_t*)A;
  a.SA = (const uint8_t*)SA;
  a.B = (const uint8_t*)B;
  a.SB = (const uint8_t*)SB;
  a.C = (_Float16*)C;
  a.M = M;
  a.N = N;
  a.K = K;
  a.nblk = K / 32;
  a.relu = relu ? 1 : 0;
  a.a_row_bytes = kind == KIND_E4M3 ? K : (kind == KIND_E2M1 ? K / 2 : 2 * (int64_t)K);
#define MX_TILE(ID, BM, BN, WGM, WGN)                                             \
  case ID:                                                                        \
    if (kind == KIND_E4M3) return launch<KIND_E4M3, BM, BN, WGM, WGN>(a, stream); \
    if (kind == KIND_E2M1) return launch<KIND_E2M1, BM, BN, WGM, WGN>(a, stream); \
    return launch<KIND_F16, BM, BN, WGM, WGN>(a, stream);
  switch (tile_id) {
    MX_TILE(0, 256, 256, 2, 2)
    MX_TILE(1, 256, 224, 2, 2)
    MX_TILE(2, 128, 128, 2, 2)
    MX_TILE(3, 64, 64, 2, 2)
    MX_TILE(4, 256, 256, 4, 2)
    MX_TILE(5, 256, 224, 4, 2)
    case 6:
      if (kind == KIND_F16) return launch<KIND_F16, 256, 256, 4, 2>(a, stream);
      return kind == KIND_E4M3 ? launch_pp<KIND_E4M3, 256, 256>(a, stream) : launch_pp<KIND_E2M1, 256, 256>(a, stream);
    case 7:
      if (kind == KIND_F16) return launch<KIND_F16, 256, 224, 4, 2>(a, stream);
      return kind == KIND_E4M3 ? launch_pp<KIND_E4M3, 256, 224>(a, stream) : launch_pp<KIND_E2M1, 256, 224>(a, stream);
    case 8:  // 4-stage ring (N % 4 == 0; K % 512 == 0 E4M3, K % 1024 == 0 E2M1; fp16: N % 256 == 0,
             // K % 256 == 0, 2KN < 2^31); otherwise the 8-wave kernel
      if (kind == KIND_E4M3 && K % 512 == 0 && N % 4 == 0) return gemm_ring_launch(0, 256, 0, 0, A, SA, B, SB, C, M, N, K, relu, stream);
      if (kind == KIND_E2M1 && K % 1024 == 0 && N % 4 == 0) return gemm_ring_launch(1, 256, 0, 0, A, SA, B, SB, C, M, N, K, relu, stream);
      if (kind == KIND_F16 && K % 256 == 0 && N % 256 == 0 && 2 * (int64_t)K * N < ((int64_t)1 << 31))
        return gemm_ring_launch(4, 256, 0, 0, A, SA, B, SB, C, M, N, K, relu, stream);
      if (kind == KIND_E4M3) return launch<KIND_E4M3, 256, 256, 4, 2>(a, stream);
      if (kind == KIND_E2M1) return launch<KIND_E2M1, 256, 256, 4, 2>(a, stream);
      return launch<KIND_F16, 256, 256, 4, 2>(a, stream);
    case 9:  // the same ring with 256x224 tiles; otherwise the 8-wave 256x224 kernel
      if (kind == KIND_E4M3 && K % 512 == 0 && N % 4 == 0) return gemm_ring_launch(0, 224, 0, 0, A, SA, B, SB, C, M, N, K, relu, stream);
      if (kind == KIND_E2M1 && K % 1024 == 0 && N % 4 == 0) return gemm_ring_launch(1, 224, 0, 0, A, SA, B, SB, C, M, N, K, relu, stream);
      if (kind == KIND_E4M3) return launch<KIND_E4M3, 256, 224, 4, 2>(a, stream);
      if (kind == KIND_E2M1) return launch<KIND_E2M1, 256, 224, 4, 2>(a, stream);
      return launch<KIND_F16, 256, 224, 4, 2>(a, stream);
    case 10:  // the ring with 256x192 tiles (E4M3 / E2M1 on the ring's shapes); otherwise the 8-wave 256x256 kernel
      if (kind == KIND_E4M3 && K % 512 == 0 && N % 4 == 0) return gemm_ring_launch(0, 192, 0, 0, A, SA, B, SB, C, M, N, K, relu, stream);
      if (kind == KIND_E2M1 && K % 1024 == 0 && N % 4 == 0) return gemm_ring_launch(1, 192, 0, 0, A, SA, B, SB, C, M, N, K, relu, stream);
      if (kind == KIND_E4M3) return launch<KIND_E4M3, 256, 256, 4, 2>(a, stream);
      if (kind == KIND_E2M1) return launch<KIND_E2M1, 256, 256, 4, 2>(a, stream);
      return launch<KIND_F16, 256, 256, 4, 2>(a, stream);
    case 11:  // 8-wave ping-pong ring, 256x256 (E4M3 or E2M1 here, K % 1024 == 0, N % 4 == 0; fp16: K % 512 == 0,
              // N % 8 == 0, 2KN < 2^31); otherwise the 4-stage ring where it applies, else the 8-wave 256x256 kernel
      if ((kind == KIND_E4M3 || kind == KIND_E2M1) && K % 1024 == 0 && N % 4 == 0)
        return gemm_pp_ring_launch(kind == KIND_E4M3 ? 0 : 1, 0, 0, A, SA, B, SB, C, M, N, K, relu, false, stream);
      if (kind == KIND_F16 && K % 512 == 0 && N % 8 == 0 && 2 * (int64_t)K * N < ((int64_t)1 << 31))
        return gemm_pp_ring_launch(4, 0, 0, A, SA, B, SB, C, M, N, K, relu, false, stream);
      if (kind == KIND_E4M3 && K % 512 == 0 && N % 4 == 0) return gemm_ring_launch(0, 256, 0, 0, A, SA, B, SB, C, M, N, K, relu, stream);
      if (kind == KIND_F16 && K % 256 == 0 && N % 256 == 0 && 2 * (int64_t)K * N < ((int64_t)1 << 31))
        return gemm_ring_launch(4, 256, 0, 0, A, SA, B, SB, C, M, N, K, relu, stream);
      if (kind == KIND_E4M3) return launch<KIND_E4M3, 256, 256, 4, 2>(a, stream);
      if (kind == KIND_E2M1) return launch<KIND_E2M1, 256, 256, 4, 2>(a, stream);
      return launch<KIND_F16, 256, 256, 4, 2>(a, stream);
    default: return MX_ERR_FORMAT;
  }
#undef MX_TILE
}

}  // namespace mx
