// mxgemm.hip -- block-scaled (MX) GEMM and fp16 GEMM kernels for gfx950.
//
// Computes C[M,N] (fp16) = A[M,K] * B[K,N] with fp32 accumulation, where for MX operands every
// 32 consecutive K-elements of a row of A (or of a column of B) share one E8M0 scale ("TensorOps
// ... notes", sections "Scale planes" and "Kernel-phase findings"; WWDC26 session 330 summary,
// section on slicing and the quantized matmul2d). The scales are applied inside the matrix core
// by the CDNA4 scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4): no dequantised copy of any
// operand exists anywhere.
//
// Structure of one workgroup (256 threads = 4 waves in a 2x2 arrangement):
//  - Output tile BM x BN; each wave owns (BM/2) x (BN/2) as 16x16 MFMA fragments whose fp32
//    accumulators stay in registers for the whole K loop.
//  - K advances in stages of 128 bytes per operand row (128 E4M3 / 256 E2M1 / 64 fp16 elements).
//    Two LDS buffers alternate. The copy of stage s+1 is issued with direct global->LDS loads
//    (global_load_lds_dwordx4 / _dword: no staging registers, no LDS write instructions) before
//    the MFMAs of stage s, so it is in flight while they run; one wait + barrier ends a stage.
//    Only a K-tail stage (K not a multiple of the stage), an unaligned scale plane, or the fp16
//    right operand (which needs a transpose) take a register path instead.
//  - LDS rows are 128 bytes = 8 chunks of 16 bytes; chunk c of row r is stored at chunk
//    c ^ ((r ^ (r >> 3)) & 7), so the 16 rows read by one fragment load hit distinct banks. A
//    direct load writes 64 lanes x 16 bytes = 8 whole rows, so each lane fetches the logical
//    chunk that lands at its physical slot.
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

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRowBytes = 128;  // bytes of one operand row per pipeline stage

MX_DEV int swz(int row) { return (row ^ (row >> 3)) & 7; }
MX_DEV int lds_off(int row, int chunk) { return row * kRowBytes + ((chunk ^ swz(row)) << 4); }

template <int KIND, int BM_, int BN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int KSTEP = KIND == KIND_E4M3 ? 128 : (KIND == KIND_E2M1 ? 256 : 64);
  static constexpr int NSB = KSTEP / 32;  // E8M0 bytes per row per stage
  static constexpr int TILE_BYTES = (BM + BN) * kRowBytes;
  static constexpr int SCALE_DW = KIND == KIND_F16 ? 0 : (BM + BN) * NSB / 4;  // scale dwords per stage
  static constexpr int STAGE_BYTES = TILE_BYTES + 4 * SCALE_DW;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  // direct loads: one wave instruction moves 8 rows (16 B per lane) or 64 scale dwords
  static constexpr int A_INSTR = BM / 8 / kWaves;
  static constexpr int B_INSTR = KIND == KIND_F16 ? 0 : BN / 8 / kWaves;
  static constexpr int S_INSTR = (SCALE_DW + 63) / 64;  // spread over the waves
  // register path (tail stage / fp16 right operand)
  static constexpr int A_CHUNKS = BM * 8 / kThreads;
  static constexpr int B_CHUNKS = KIND == KIND_F16 ? 0 : BN * 8 / kThreads;
  static constexpr int B_MICRO = KIND == KIND_F16 ? (BN + kThreads - 1) / kThreads : 0;  // 8x8 fp16 blocks
  static_assert(BM % 32 == 0 && BN % 32 == 0, "tile");
  static_assert((BM / 8) % kWaves == 0 && (KIND == KIND_F16 || (BN / 8) % kWaves == 0), "direct loads");
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
};

MX_DEV void g2l(const void* g, char* lds_wave_base, int size) {
  if (size == 16)
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)g, (lds_ptr_t)lds_wave_base, 16, 0, 0);
  else
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)g, (lds_ptr_t)lds_wave_base, 4, 0, 0);
}

// Direct copy of the code rows of stage s (A, and B for MX kinds) into one LDS stage buffer.
template <class CF, int KIND>
MX_DEV void issue_direct_rows(const Args& p, char* buf, int m0, int n0, int s, int wave, int lane) {
  const int64_t kbyte0 = (int64_t)s * kRowBytes;
  const int rsub = lane >> 3, pch = lane & 7;
#pragma unroll
  for (int i = 0; i < CF::A_INSTR; i++) {
    const int r0 = (wave * CF::A_INSTR + i) * 8, row = r0 + rsub;
    const int gr = min(m0 + row, p.M - 1);
    const uint8_t* g = p.A + (int64_t)gr * p.a_row_bytes + kbyte0 + ((pch ^ swz(row)) << 4);
    g2l(g, buf + r0 * kRowBytes, 16);
  }
#pragma unroll
  for (int i = 0; i < CF::B_INSTR; i++) {
    const int r0 = (wave * CF::B_INSTR + i) * 8, row = r0 + rsub;
    const int gr = min(n0 + row, p.N - 1);
    const uint8_t* g = p.B + (int64_t)gr * p.a_row_bytes + kbyte0 + ((pch ^ swz(CF::BM + row)) << 4);
    g2l(g, buf + (CF::BM + r0) * kRowBytes, 16);
  }
}

// Direct copy of the stage's scale dwords (A rows then B rows, NSB bytes each); needs K/32 % 4 == 0.
template <class CF>
MX_DEV void issue_direct_scales(const Args& p, char* buf, int m0, int n0, int s, int wave, int lane) {
  constexpr int per_row = CF::NSB / 4;
#pragma unroll
  for (int i = wave; i < CF::S_INSTR; i += kWaves) {
    const int did = i * 64 + lane;
    if (did < CF::SCALE_DW) {
      const int row = did / per_row, dw = did % per_row;
      const bool isA = row < CF::BM;
      const int gr = isA ? min(m0 + row, p.M - 1) : min(n0 + row - CF::BM, p.N - 1);
      const uint8_t* g = (isA ? p.SA : p.SB) + (int64_t)gr * p.nblk + s * CF::NSB + 4 * dw;
      g2l(g, buf + CF::TILE_BYTES + i * 256, 4);
    }
  }
}

// Register path for one stage: zero-filled codes past K, scale 127 (= 1.0) for blocks past K.
template <class CF, int KIND>
MX_DEV void copy_stage_regs(const Args& p, char* buf, int m0, int n0, int s, int tid, bool rows, bool scales) {
  const int64_t kbyte0 = (int64_t)s * kRowBytes;
  if (rows) {
#pragma unroll
    for (int i = 0; i < CF::A_CHUNKS; i++) {
      const int cid = tid + kThreads * i, row = cid >> 3, cc = cid & 7;
      const int gr = min(m0 + row, p.M - 1);
      const int64_t kb = kbyte0 + cc * 16;
      const v4i v = kb < p.a_row_bytes ? *reinterpret_cast<const v4i*>(p.A + (int64_t)gr * p.a_row_bytes + kb)
                                       : v4i{0, 0, 0, 0};
      *reinterpret_cast<v4i*>(buf + lds_off(row, cc)) = v;
    }
#pragma unroll
    for (int i = 0; i < CF::B_CHUNKS; i++) {
      const int cid = tid + kThreads * i, row = cid >> 3, cc = cid & 7;
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
      for (int did = tid; did < CF::SCALE_DW; did += kThreads) {
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
    const int mb = tid + kThreads * u;
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
    const int mb = tid + kThreads * u;
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

template <class CF, int KIND>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(Args p) {
  __shared__ __attribute__((aligned(16))) char lds[CF::LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
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
  auto start_stage = [&](int s, char* buf) {
    const bool full = (int64_t)(s + 1) * kRowBytes <= p.a_row_bytes;
    if (full) issue_direct_rows<CF, KIND>(p, buf, m0, n0, s, wave, lane);
    if constexpr (KIND != KIND_F16) {
      if (full && aligned_scales) issue_direct_scales<CF>(p, buf, m0, n0, s, wave, lane);
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
    __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads have landed in LDS
    __syncthreads();                // ... and every other wave's
  }

  // Epilogue: fp32 -> fp16 (nearest even), lane holds C[m][n..n+3].
  const bool vec = (p.N & 3) == 0;
#pragma unroll
  for (int i = 0; i < CF::FN; i++) {
    const int n = n0 + wn * CF::WN + 16 * i + 4 * q;
#pragma unroll
    for (int j = 0; j < CF::FM; j++) {
      const int m = m0 + wm * CF::WM + 16 * j + r16;
      if (m >= p.M) continue;
      _Float16* crow = p.C + (int64_t)m * p.N;
      const v4f a = acc[i][j];
      if (vec && n + 3 < p.N) {
        *reinterpret_cast<v4h*>(crow + n) = v4h{(_Float16)a[0], (_Float16)a[1], (_Float16)a[2], (_Float16)a[3]};
      } else {
#pragma unroll
        for (int v = 0; v < 4; v++)
          if (n + v < p.N) crow[n + v] = (_Float16)a[v];
      }
    }
  }
}

template <int KIND, int BM, int BN>
int launch(const Args& a0, hipStream_t stream) {
  using CF = Cfg<KIND, BM, BN>;
  Args a = a0;
  a.tiles_m = (a.M + BM - 1) / BM;
  a.tiles_n = (a.N + BN - 1) / BN;
  a.nstages = (int)((a.a_row_bytes + kRowBytes - 1) / kRowBytes);
  const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
  if (tiles > 0x7FFFFFFF) return MX_ERR_SHAPE;
  hipLaunchKernelGGL((gemm_kernel<CF, KIND>), dim3((unsigned)tiles), dim3(kThreads), 0, stream, a);
  return mx::launch_status();
}

}  // namespace

namespace mx {

// Tile configurations, indexed by the plan. Returns MX_ERR_FORMAT for an unknown id.
int gemm_launch(int kind, int tile_id, const void* A, const void* SA, const void* B, const void* SB, void* C, int M,
                int N, int K, hipStream_t stream) {
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
  a.a_row_bytes = kind == KIND_E4M3 ? K : (kind == KIND_E2M1 ? K / 2 : 2 * (int64_t)K);
#define MX_TILE(ID, BM, BN)                                             \
  case ID:                                                              \
    if (kind == KIND_E4M3) return launch<KIND_E4M3, BM, BN>(a, stream); \
    if (kind == KIND_E2M1) return launch<KIND_E2M1, BM, BN>(a, stream); \
    return launch<KIND_F16, BM, BN>(a, stream);
  switch (tile_id) {
    MX_TILE(0, 256, 256)
    MX_TILE(1, 256, 224)
    MX_TILE(2, 128, 128)
    MX_TILE(3, 64, 64)
    default: return MX_ERR_FORMAT;
  }
#undef MX_TILE
}

}  // namespace mx
