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
//  - Output tile BM x BN, each wave owns (BM/2) x (BN/2) as 16x16 MFMA fragments whose fp32
//    accumulators stay in registers for the whole K loop.
//  - K advances in stages of 128 bytes per operand row (128 E4M3 / 256 E2M1 / 64 fp16 elements).
//    A stage of A (BM rows) and B (BN rows, K-contiguous) plus their E8M0 scale bytes is copied
//    global -> registers -> LDS with 16-byte loads; two LDS buffers alternate, so the loads of
//    stage s+1 are in flight while the MFMAs of stage s run, with one barrier per stage.
//  - LDS rows are 128 bytes = 8 chunks of 16 bytes; chunk c of row r is stored at chunk
//    c ^ ((r ^ (r >> 3)) & 7), so the 16 rows read by one fragment load hit distinct banks.
//  - The MFMA's first operand is the B fragment and its second the A fragment, so each lane ends
//    with 4 consecutive n of one output row m and writes them with one 8-byte store.
//  - Workgroup ids are remapped so that each of the 8 XCDs (private L2 each) works on a
//    contiguous range of tiles; tiles are ordered m-fastest, so concurrently running tiles on an
//    XCD share their B panel and the A panel of the whole problem's K-window stays L2-resident.
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

enum Kind { KIND_E4M3 = 0, KIND_E2M1 = 1, KIND_F16 = 2 };

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;  // bytes of one operand row per pipeline stage

MX_DEV int lds_off(int row, int chunk) { return row * kRowBytes + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4); }

template <int KIND, int BM_, int BN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int KSTEP = KIND == KIND_E4M3 ? 128 : (KIND == KIND_E2M1 ? 256 : 64);
  static constexpr int NSB = KSTEP / 32;  // E8M0 bytes per row per stage
  static constexpr int TILE_BYTES = (BM + BN) * kRowBytes;
  static constexpr int SCALE_BYTES = KIND == KIND_F16 ? 0 : (BM + BN) * NSB;
  static constexpr int STAGE_BYTES = TILE_BYTES + SCALE_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static constexpr int A_CHUNKS = BM * 8 / kThreads;
  static constexpr int B_CHUNKS = KIND == KIND_F16 ? 0 : BN * 8 / kThreads;
  static constexpr int B_MICRO = KIND == KIND_F16 ? (BN + kThreads - 1) / kThreads : 0;  // 8x8 fp16 blocks
  static constexpr int S_DWORDS = KIND == KIND_F16 ? 0 : ((BM + BN) * NSB / 4 + kThreads - 1) / kThreads;
  static_assert(BM % 32 == 0 && BN % 32 == 0, "tile");
  static_assert((BM * 8) % kThreads == 0 && (KIND == KIND_F16 || (BN * 8) % kThreads == 0), "chunks");
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

// Per-thread registers holding one stage in flight from global memory.
template <class CF, int KIND>
struct Stage {
  v4i a[CF::A_CHUNKS];
  v4i b[KIND == KIND_F16 ? 1 : CF::B_CHUNKS];
  v4i bt[KIND == KIND_F16 ? CF::B_MICRO * 8 : 1];
  uint32_t s[CF::S_DWORDS > 0 ? CF::S_DWORDS : 1];
};

template <class CF, int KIND>
MX_DEV void load_stage(Stage<CF, KIND>& st, const Args& p, int m0, int n0, int s, int tid, bool fast_scales) {
  const int64_t kbyte0 = (int64_t)s * kRowBytes;
#pragma unroll
  for (int i = 0; i < CF::A_CHUNKS; i++) {
    const int cid = tid + kThreads * i, row = cid >> 3, cc = cid & 7;
    const int gr = min(m0 + row, p.M - 1);
    const int64_t kb = kbyte0 + cc * 16;
    st.a[i] = kb < p.a_row_bytes ? *reinterpret_cast<const v4i*>(p.A + (int64_t)gr * p.a_row_bytes + kb) : v4i{0, 0, 0, 0};
  }
  if constexpr (KIND != KIND_F16) {
#pragma unroll
    for (int i = 0; i < CF::B_CHUNKS; i++) {
      const int cid = tid + kThreads * i, row = cid >> 3, cc = cid & 7;
      const int gr = min(n0 + row, p.N - 1);
      const int64_t kb = kbyte0 + cc * 16;
      st.b[i] = kb < p.a_row_bytes ? *reinterpret_cast<const v4i*>(p.B + (int64_t)gr * p.a_row_bytes + kb) : v4i{0, 0, 0, 0};
    }
    // E8M0 scales of this stage: NSB bytes per row, A rows then B rows. Blocks past K read as
    // 127 (scale 1) with zero codes, so they contribute exactly nothing.
    const int blk0 = s * CF::NSB;
#pragma unroll
    for (int i = 0; i < CF::S_DWORDS; i++) {
      const int did = tid + kThreads * i;
      const int per_row = CF::NSB / 4;
      const int row = did / per_row, dw = did % per_row;
      uint32_t v = 0x7F7F7F7Fu;
      if (row < CF::BM + CF::BN) {
        const bool isA = row < CF::BM;
        const int gr = isA ? min(m0 + row, p.M - 1) : min(n0 + row - CF::BM, p.N - 1);
        const uint8_t* srow = (isA ? p.SA : p.SB) + (int64_t)gr * p.nblk;
        const int b = blk0 + 4 * dw;
        if (fast_scales) {
          if (b < p.nblk) v = *reinterpret_cast<const uint32_t*>(srow + b);
        } else {
          v = 0u;
#pragma unroll
          for (int j = 0; j < 4; j++) v |= (uint32_t)(b + j < p.nblk ? srow[b + j] : 127u) << (8 * j);
        }
      }
      st.s[i] = v;
    }
  } else {
    // fp16 B is [K][N] row-major: each thread reads an 8 (k) x 8 (n) block with eight 16-byte
    // row loads; it is transposed in registers before the LDS store.
#pragma unroll
    for (int u = 0; u < CF::B_MICRO; u++) {
      const int mb = tid + kThreads * u;
      const int nchunks = CF::BN / 8;
      const int nc = mb % nchunks, kg = mb / nchunks;
      const int n = n0 + nc * 8;
#pragma unroll
      for (int r = 0; r < 8; r++) {
        const int k = s * 64 + kg * 8 + r;
        const bool ok = mb < CF::BN && k < p.K && n < p.N;
        st.bt[u * 8 + r] = ok ? *reinterpret_cast<const v4i*>(p.B + ((int64_t)k * p.N + n) * 2) : v4i{0, 0, 0, 0};
      }
    }
  }
}

template <class CF, int KIND>
MX_DEV void store_stage(const Stage<CF, KIND>& st, char* lds, int tid) {
#pragma unroll
  for (int i = 0; i < CF::A_CHUNKS; i++) {
    const int cid = tid + kThreads * i;
    *reinterpret_cast<v4i*>(lds + lds_off(cid >> 3, cid & 7)) = st.a[i];
  }
  if constexpr (KIND != KIND_F16) {
#pragma unroll
    for (int i = 0; i < CF::B_CHUNKS; i++) {
      const int cid = tid + kThreads * i;
      *reinterpret_cast<v4i*>(lds + lds_off(CF::BM + (cid >> 3), cid & 7)) = st.b[i];
    }
    uint32_t* sl = reinterpret_cast<uint32_t*>(lds + CF::TILE_BYTES);
#pragma unroll
    for (int i = 0; i < CF::S_DWORDS; i++) {
      const int did = tid + kThreads * i;
      if (did < (CF::BM + CF::BN) * CF::NSB / 4) sl[did] = st.s[i];
    }
  } else {
#pragma unroll
    for (int u = 0; u < CF::B_MICRO; u++) {
      const int mb = tid + kThreads * u;
      if (mb >= CF::BN) break;
      const int nchunks = CF::BN / 8;
      const int nc = mb % nchunks, kg = mb / nchunks;
      // transpose 8x8 halves: out[j] = 8 k-values of column n = nc*8 + j
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int p2 = j >> 1;
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        v4i o;
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const uint32_t lo = (uint32_t)st.bt[u * 8 + 2 * q][p2], hi = (uint32_t)st.bt[u * 8 + 2 * q + 1][p2];
          o[q] = (int)__builtin_amdgcn_perm(hi, lo, sel);
        }
        *reinterpret_cast<v4i*>(lds + lds_off(CF::BM + nc * 8 + j, kg)) = o;
      }
    }
  }
}

MX_DEV v4i lds_read16(const char* lds, int row, int chunk) {
  return *reinterpret_cast<const v4i*>(lds + lds_off(row, chunk));
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
  const bool fast_scales = (p.nblk & 3) == 0;

  v4f acc[CF::FN][CF::FM];
#pragma unroll
  for (int i = 0; i < CF::FN; i++)
#pragma unroll
    for (int j = 0; j < CF::FM; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  Stage<CF, KIND> st;
  load_stage<CF, KIND>(st, p, m0, n0, 0, tid, fast_scales);
  store_stage<CF, KIND>(st, lds, tid);
  __syncthreads();

  for (int s = 0; s < p.nstages; s++) {
    const bool more = s + 1 < p.nstages;
    if (more) load_stage<CF, KIND>(st, p, m0, n0, s + 1, tid, fast_scales);
    const char* buf = lds + (s & 1) * CF::STAGE_BYTES;
    const uint8_t* sc = reinterpret_cast<const uint8_t*>(buf + CF::TILE_BYTES);

    if constexpr (KIND == KIND_E4M3) {
      v8i af[CF::FM];
      int sa[CF::FM];
#pragma unroll
      for (int j = 0; j < CF::FM; j++) {
        const int row = wm * CF::WM + 16 * j + r16;
        const v4i x0 = lds_read16(buf, row, q), x1 = lds_read16(buf, row, 4 + q);
        af[j] = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        sa[j] = sc[row * CF::NSB + q];
      }
#pragma unroll
      for (int i = 0; i < CF::FN; i++) {
        const int row = CF::BM + wn * CF::WN + 16 * i + r16;
        const v4i x0 = lds_read16(buf, row, q), x1 = lds_read16(buf, row, 4 + q);
        const v8i bf = v8i{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        const int sb = sc[row * CF::NSB + q];
#pragma unroll
        for (int j = 0; j < CF::FM; j++)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[j], acc[i][j], 0, 0, 0, sb, 0, sa[j]);
      }
    } else if constexpr (KIND == KIND_E2M1) {
      v4i af[2][CF::FM];
      int sa[CF::FM];
#pragma unroll
      for (int j = 0; j < CF::FM; j++) {
        const int row = wm * CF::WM + 16 * j + r16;
        af[0][j] = lds_read16(buf, row, q);
        af[1][j] = lds_read16(buf, row, 4 + q);
        sa[j] = sc[row * CF::NSB + q] | (sc[row * CF::NSB + 4 + q] << 8);
      }
#pragma unroll
      for (int i = 0; i < CF::FN; i++) {
        const int row = CF::BM + wn * CF::WN + 16 * i + r16;
        const v4i b0 = lds_read16(buf, row, q), b1 = lds_read16(buf, row, 4 + q);
        const int sb = sc[row * CF::NSB + q] | (sc[row * CF::NSB + 4 + q] << 8);
        const v8i bf0 = v8i{b0[0], b0[1], b0[2], b0[3], 0, 0, 0, 0};
        const v8i bf1 = v8i{b1[0], b1[1], b1[2], b1[3], 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < CF::FM; j++) {
          const v8i a0 = v8i{af[0][j][0], af[0][j][1], af[0][j][2], af[0][j][3], 0, 0, 0, 0};
          const v8i a1 = v8i{af[1][j][0], af[1][j][1], af[1][j][2], af[1][j][3], 0, 0, 0, 0};
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf0, a0, acc[i][j], 4, 4, 0, sb, 0, sa[j]);
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf1, a1, acc[i][j], 4, 4, 1, sb, 1, sa[j]);
        }
      }
    } else {
      v8h af[2][CF::FM];
#pragma unroll
      for (int j = 0; j < CF::FM; j++) {
        const int row = wm * CF::WM + 16 * j + r16;
        af[0][j] = __builtin_bit_cast(v8h, lds_read16(buf, row, q));
        af[1][j] = __builtin_bit_cast(v8h, lds_read16(buf, row, 4 + q));
      }
#pragma unroll
      for (int i = 0; i < CF::FN; i++) {
        const int row = CF::BM + wn * CF::WN + 16 * i + r16;
        const v8h b0 = __builtin_bit_cast(v8h, lds_read16(buf, row, q));
        const v8h b1 = __builtin_bit_cast(v8h, lds_read16(buf, row, 4 + q));
#pragma unroll
        for (int j = 0; j < CF::FM; j++) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b0, af[0][j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b1, af[1][j], acc[i][j], 0, 0, 0);
        }
      }
    }

    if (more) store_stage<CF, KIND>(st, lds + ((s + 1) & 1) * CF::STAGE_BYTES, tid);
    __syncthreads();
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
        typedef _Float16 v4h __attribute__((ext_vector_type(4)));
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
  if (KIND == KIND_F16) a.nstages = (a.K + 63) / 64;
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
#define MX_TILE(ID, BM, BN)                                           \
  case ID:                                                            \
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
