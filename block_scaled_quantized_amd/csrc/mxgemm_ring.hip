// mxgemm_ring.hip -- MXFP8 / MXFP4 (E4M3 or E2M1 data, E8M0 scales per 32 along K) GEMM with a
// 4-stage LDS ring.
//
//   C[m,n] = sum_k 2^(SA[m,k/32]-127) A[m,k] * 2^(SB[n,k/32]-127) B[n,k]   (fp32 accumulate, fp16 out)
//
// the block-scaled product of "TensorOps ... notes", sections "Scale planes" and "Kernel-phase
// findings", with the E8M0 scale plane of the WWDC26 session 330 summary; B is K-contiguous.
//
// Why a ring of short stages: a 256x224 tile with 128-byte K stages fills LDS with two stages, so
// each stage's copy has to land within one stage of MFMAs (about 1800 cycles), less than the L2 /
// MALL latency under load. Here a stage is 64 bytes of K: one scaled MFMA 32x32x64 deep for E4M3,
// two for E2M1.
//  - Tile 256 x 256 with 4 waves (one per SIMD) of 128 x 128 = 4 x 4 MFMA tiles of 32 x 32, or
//    256 x 224 with 4 waves of 64 x 224 = 2 x 7 MFMA tiles (224 = 7 x 32 does not split in two:
//    the 256 x 224 tile exists so that N = 14336 gives 64 column tiles, a whole number of rounds
//    on 256 CUs at M = 2048).
//  - LDS ring of 4 stages (4 separate arrays, so the compiler can tell a fragment read of one
//    stage from the direct copies filling another): up to 256 + 256 rows x 64 bytes per stage.
//    Copies for stage t+3 are queued while stage t computes, three stages ahead.
//  - 64-byte rows hold four 16-byte chunks, stored at chunk ^ ((row >> 2) & 3): a 16-lane quarter of
//    a fragment read (16 rows, one chunk) then covers all 64 banks once.
//  - Direct global->LDS copies (16 bytes per lane): instruction i of a stage fills rows
//    16i..16i+15; lane l fills physical chunk l%4 of row 16i + l/4. Each wave issues 8 per stage;
//    instructions past the tile's rows get an empty buffer resource and fill unused slot bytes
//    with zeros, so every wave's copy count (and its vmcnt bookkeeping) is the same.
//  - E8M0 scales for 8 stages (16 / 32 bytes per row) are copied once per group into the scale
//    array (after every wave has read the previous group's); each lane packs its own K-block's
//    bytes so that byte u%4 of dword u/4 is its scale for K-step u of the group (op_sel picks the
//    byte).
//  - Fragments of stage t+1 are read from LDS while the MFMAs of stage t run; one barrier per
//    stage, after this wave's copies of stage t+1 have landed (vmcnt), publishes stage t+1 and
//    frees the slot of stage t-1.
// Operand layout of v_mfma_scale_f32_32x32x64_f8f6f4 (measured): lane l feeds row l%32 and, with
// h = l/32, E4M3 K bytes 16h..16h+15 and 32+16h..32+16h+15, or E2M1 elements 32h..32h+31 (16
// bytes); it supplies the scale of (row l%32, K-block h); output element e of lane l is row
// 8(e/4) + 4h + e%4 of the first operand and column l%32 of the second. B is the first operand, so
// each lane ends with 4 consecutive n of one row m.
#include <type_traits>

#include "common.h"

namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int BM = 256;                 // tile rows (both shapes)
constexpr int ROWB = 64;                // K bytes per stage
constexpr int SLOT = 512 * ROWB;        // 32 KB: room for 256 + 256 rows
constexpr int GROUP = 8;                // stages per scale group
constexpr int DMA_PER_STAGE = SLOT / 1024 / 4;  // direct copies per wave per stage (8)

// Tile shapes. WAVES_M waves along M (the rest along N); each wave holds FA x FB MFMA tiles of
// 32 x 32 (FA along M, FB along N).
template <int WAVES_M_>
struct RingTile {
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = 4 / WAVES_M;
  static constexpr int BN = WAVES_M == 2 ? 256 : 224;
  static constexpr int FA = BM / 32 / WAVES_M, FB = BN / 32 / WAVES_N;
  static constexpr int F = FA + FB;  // fragments read per stage per wave
  static_assert(WAVES_M == 2 || WAVES_M == 4, "tile");
};

// Per-format constants. A 64-byte stage is one MFMA K-step of E4M3 (64 elements, 2 scale blocks)
// or two of E2M1 (128 elements, 4 blocks); a group of 8 stages then holds 16 or 32 scale bytes per
// row, and each lane keeps 8 or 16 of them (its own K-block h of every K-step), 2 or 4 dwords.
template <int KIND>
struct RingFmt {
  static constexpr bool FP4 = KIND == 1;
  static constexpr int KSTEPS = FP4 ? 2 : 1;        // MFMA K-steps per stage
  static constexpr int SGRP = 512 * 16 * KSTEPS;    // scale array: 8 / 16 KB
  static constexpr int SDW = 2 * KSTEPS;            // packed scale dwords per row per lane
  static constexpr int DMA_PER_GROUP = SGRP / 1024 / 4;  // scale copies per wave per group (2 / 4)
  static constexpr int ELEMS_PER_BYTE = FP4 ? 2 : 1;
};

// The size goes through readfirstlane: clamps of uniform values can be selected as vector ops
// (v_med3), and a resource that is not provably scalar turns each buffer access into a loop.
MX_DEV rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}
MX_DEV void raw_barrier() { asm volatile("s_barrier" ::: "memory"); }

// vmcnt(n), other counters untouched (gfx9 s_waitcnt encoding); n <= 31 here.
MX_DEV void wait_vm_n(int n) {
  switch (n) {
#define MX_W(k) \
  case k: __builtin_amdgcn_s_waitcnt(((k) & 0xF) | 0x0F70 | ((((k) >> 4) & 3) << 14)); break;
    MX_W(0) MX_W(1) MX_W(2) MX_W(3) MX_W(4) MX_W(5) MX_W(6) MX_W(7) MX_W(8) MX_W(9) MX_W(10) MX_W(11)
    MX_W(12) MX_W(13) MX_W(14) MX_W(15) MX_W(16) MX_W(17) MX_W(18) MX_W(19) MX_W(20) MX_W(21) MX_W(22)
    MX_W(23) MX_W(24) MX_W(25) MX_W(26) MX_W(27) MX_W(28) MX_W(29) MX_W(30) MX_W(31)
#undef MX_W
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
}

struct Args {
  const uint8_t* A;
  const uint8_t* SA;
  const uint8_t* B;
  const uint8_t* SB;
  _Float16* C;
  int M, N, K, tiles_m;
  int relu;  // epilogue: C = max(C, 0) (IEEE maxNum: NaN gives 0)
};

// Per lane: byte u%4 of dword u/4 is the lane's scale for MFMA K-step u of the group (u = stage for
// E4M3, 2*stage + k for K-step k of a stage for E2M1).
template <int KIND, class T>
struct Scales {
  uint32_t a[T::FA][RingFmt<KIND>::SDW], b[T::FB][RingFmt<KIND>::SDW];
};

MX_DEV int phys_off(int row, int chunk) { return row * ROWB + ((chunk ^ ((row >> 2) & 3)) << 4); }

MX_DEV v4i lds16(const char* base, int off) { return *reinterpret_cast<const v4i*>(base + off); }

// Scale layout in LDS. E4M3: row r's 16 bytes of the group at r*16, (stage s, block b) at byte
// 2s + b. E2M1: two planes of 8 KB (stages 0-3, 4-7), row r's 16 bytes of plane d at d*8192 + r*16,
// (stage s, K-step k, block b) at byte 4(s%4) + 2k + b. Half d of a row covers stages 4d..4d+3
// and becomes dwords d*KSTEPS.. of the lane's packed scales, keeping its own block h: from each 8
// source bytes, bytes h, 2+h, 4+h, 6+h. Stages 0-3 of a group use the dwords of half 0 and stages
// 4-7 those of half 1, so the next group's half 0 is read during stage 4 and packed at the end of
// stage 6, and its half 1 is read after the last MFMA of stage 7 and packed at the end of the next
// group's stage 2: the reads have a stage or more to land before anything waits for them. The
// packed value of stage 2 is unchanged in group 0, whose halves the prologue packs.
template <int KIND>
struct RawT {
  typedef int type __attribute__((ext_vector_type(2 * RingFmt<KIND>::KSTEPS)));
};

template <int KIND, class T>
struct RawScales {
  typename RawT<KIND>::type a[T::FA], b[T::FB];
};

// Rows of the wave's fragments: A fragment j is LDS row 32*FA*wm + 32j + l%32, B fragment i is
// row BM + 32*FB*wn + 32i + l%32.
template <class T>
MX_DEV int row_a(int j, int wm, int r32) { return 32 * T::FA * wm + 32 * j + r32; }
template <class T>
MX_DEV int row_b(int i, int wn, int r32) { return BM + 32 * T::FB * wn + 32 * i + r32; }

template <int KIND>
MX_DEV typename RawT<KIND>::type raw_at(const char* sg, int row, int d) {
  typedef typename RawT<KIND>::type raw_t;
  if constexpr (RingFmt<KIND>::FP4) return *reinterpret_cast<const raw_t*>(sg + d * 8192 + row * 16);
  else return *reinterpret_cast<const raw_t*>(sg + row * 16 + 8 * d);
}

template <int KIND, class T>
MX_DEV void read_raw_scales(const char* sg, RawScales<KIND, T>& r, int d, int wm, int wn, int r32) {
#pragma unroll
  for (int j = 0; j < T::FA; j++) r.a[j] = raw_at<KIND>(sg, row_a<T>(j, wm, r32), d);
#pragma unroll
  for (int i = 0; i < T::FB; i++) r.b[i] = raw_at<KIND>(sg, row_b<T>(i, wn, r32), d);
}

template <int KIND, class T>
MX_DEV void pack_scales(const RawScales<KIND, T>& r, Scales<KIND, T>& s, int d, int h) {
  constexpr int KS = RingFmt<KIND>::KSTEPS;
  const uint32_t sel = h ? 0x07050301u : 0x06040200u;
#pragma unroll
  for (int w = 0; w < KS; w++) {
#pragma unroll
    for (int j = 0; j < T::FA; j++)
      s.a[j][KS * d + w] = __builtin_amdgcn_perm((uint32_t)r.a[j][2 * w + 1], (uint32_t)r.a[j][2 * w], sel);
#pragma unroll
    for (int i = 0; i < T::FB; i++)
      s.b[i][KS * d + w] = __builtin_amdgcn_perm((uint32_t)r.b[i][2 * w + 1], (uint32_t)r.b[i][2 * w], sel);
  }
}

// A fragment of one stage: chunks h and 2+h of its row, i.e. the lane's K bytes of the E4M3 MFMA,
// or its 16 bytes (K-block h) of E2M1 K-steps 0 and 1 in the low and high halves.
MX_DEV v8i read_frag(const char* slot, int row, int h) {
  return __builtin_shufflevector(lds16(slot, phys_off(row, h)), lds16(slot, phys_off(row, 2 + h)), 0, 1, 2, 3, 4, 5,
                                 6, 7);
}

// Per-workgroup constants of the main loop (rscale: the first DMA_PER_GROUP of the format are set).
struct Ctx {
  rsrc_t rdata[DMA_PER_STAGE];
  rsrc_t rscale[4];
  uint32_t voff, svoff;
  int wave, wm, wn, r32, h, nst, ngroups;
};

// Scale copy k of this wave: 64 rows (A rows 64(wave) + l for even k, B rows for odd k), 16 bytes
// each: bytes 16(k/2).. of the row's group (E2M1: plane k/2).
template <int KIND>
MX_DEV void issue_scales(const Ctx& c, char* sg, int g) {
  constexpr int NK = RingFmt<KIND>::DMA_PER_GROUP;
  const int goff = g * (RingFmt<KIND>::FP4 ? 32 : 16);  // bytes of the group's first scale
#pragma unroll
  for (int k = 0; k < NK; k++)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rscale[k], (lds_ptr_t)(sg + (c.wave + 4 * k) * 1024), 16, c.svoff,
                                             goff + 16 * (k >> 1), 0, 0);
}

// One stage t = 8g + S8: slot t%4 holds stage t (its fragments already in ca/cb). Before the
// barrier this wave's copies of stage t+1 must have landed; after it, slot (t+3)%4 (stage t-1,
// read during stage t-2) is free and stage t+1 is readable by every wave. The MFMAs go B tile by B
// tile; after each tile come its share of the 8 copies of stage t+3 and of the next stage's
// fragments, read into the other register set (dead during this stage): the A fragments first, as
// the next stage's first B tile needs all of them, then the B fragments in the order their tiles
// come. The next-stage reads are unconditional (after the last stage they fetch unused bytes): a
// conditional overwrite would keep the old contents alive through the stage.
template <int KIND, class T, int S8>
MX_DEV void ring_stage(const Ctx& c, int g, char* sgrp, const v8i (&ca)[T::FA], const v8i (&cb)[T::FB],
                       v8i (&na)[T::FA], v8i (&nb)[T::FB], const char* slot_nxt, char* slot_fill,
                       Scales<KIND, T>& sc, RawScales<KIND, T>& raw, v16f (&acc)[T::FB][T::FA]) {
  using F = RingFmt<KIND>;
  const int t = GROUP * g + S8;
  // Copies queued after this wave's copies of stage t+1 (issued at stage t-2): those of stage t+2
  // (at stage t-1) and, at S8 == 3, the scale group issued at S8 == 2 ahead of them. From S8 == 4
  // on, the next group's scales are visible.
  wait_vm_n(S8 == 3 ? DMA_PER_STAGE + F::DMA_PER_GROUP : DMA_PER_STAGE);
  raw_barrier();
  // The scale array still holds half 1 of group g, read at the end of stage 7 of group g-1. Every
  // wave has waited for those reads before stage 1's MFMAs (they precede the fragment reads of
  // stage 0 in the wave's LDS queue), so past stage 2's barrier the array is free.
  if (S8 == 2) issue_scales<KIND>(c, sgrp, min(g + 1, c.ngroups - 1));
  const uint32_t fill_off = ROWB * min(t + 3, c.nst - 1);
#pragma unroll
  for (int i = 0; i < T::FB; i++) {
#pragma unroll
    for (int k = 0; k < F::KSTEPS; k++) {
      constexpr int U0 = F::KSTEPS * S8;  // first K-step of the stage within the group
#pragma unroll
      for (int j = 0; j < T::FA; j++) {
        if constexpr (F::FP4) {
          const v8i bk = k ? __builtin_shufflevector(cb[i], cb[i], 4, 5, 6, 7, -1, -1, -1, -1)
                           : __builtin_shufflevector(cb[i], cb[i], 0, 1, 2, 3, -1, -1, -1, -1);
          const v8i ak = k ? __builtin_shufflevector(ca[j], ca[j], 4, 5, 6, 7, -1, -1, -1, -1)
                           : __builtin_shufflevector(ca[j], ca[j], 0, 1, 2, 3, -1, -1, -1, -1);
          if (k == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bk, ak, acc[i][j], 4, 4, U0 % 4, sc.b[i][U0 / 4], U0 % 4, sc.a[j][U0 / 4]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bk, ak, acc[i][j], 4, 4, (U0 + 1) % 4, sc.b[i][(U0 + 1) / 4], (U0 + 1) % 4, sc.a[j][(U0 + 1) / 4]);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cb[i], ca[j], acc[i][j], 0, 0, U0 % 4,
                                                                       sc.b[i][U0 / 4], U0 % 4, sc.a[j][U0 / 4]);
        }
      }
    }
    // this tile's share of the stage copies: copies [8i/FB, 8(i+1)/FB)
#pragma unroll
    for (int q = DMA_PER_STAGE * i / T::FB; q < DMA_PER_STAGE * (i + 1) / T::FB; q++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rdata[q], (lds_ptr_t)(slot_fill + (c.wave + 4 * q) * 1024), 16,
                                               c.voff, fill_off, 0, 0);
    // and of the next stage's fragments: list positions [F*i/FB, F*(i+1)/FB) of A0.., B0..
#pragma unroll
    for (int f = T::F * i / T::FB; f < T::F * (i + 1) / T::FB; f++) {
      if (f < T::FA) na[f] = read_frag(slot_nxt, row_a<T>(f, c.wm, c.r32), c.h);
      else nb[f - T::FA] = read_frag(slot_nxt, row_b<T>(f - T::FA, c.wn, c.r32), c.h);
    }
    if (S8 == 4 && i == 1) read_raw_scales<KIND, T>(sgrp, raw, 0, c.wm, c.wn, c.r32);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (S8 == 2) pack_scales<KIND, T>(raw, sc, 1, c.h);
  if (S8 == 6) pack_scales<KIND, T>(raw, sc, 0, c.h);
  if (S8 == GROUP - 1) read_raw_scales<KIND, T>(sgrp, raw, 1, c.wm, c.wn, c.r32);
}

template <int KIND, int WAVES_M>
__global__ __launch_bounds__(256, 1) void gemm_ring_kernel(Args p) {
  using F = RingFmt<KIND>;
  using T = RingTile<WAVES_M>;
  constexpr int BN = T::BN;
  __shared__ __attribute__((aligned(16))) char slot0[SLOT];
  __shared__ __attribute__((aligned(16))) char slot1[SLOT];
  __shared__ __attribute__((aligned(16))) char slot2[SLOT];
  __shared__ __attribute__((aligned(16))) char slot3[SLOT];
  __shared__ __attribute__((aligned(16))) char sgrp[F::SGRP];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % T::WAVES_M, wn = wave / T::WAVES_M;
  const int r32 = lane & 31, h = lane >> 5;

  int bid = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);  // each XCD takes a contiguous tile range
  const int tm = bid % p.tiles_m, tn = bid / p.tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int rows_a = min(BM, p.M - m0), rows_b = min(BN, p.N - n0);
  const uint32_t RB = (uint32_t)p.K / F::ELEMS_PER_BYTE, nblk = (uint32_t)p.K / 32;  // row bytes, K-blocks
  const int nst = (int)RB / ROWB, ngroups = nst / GROUP;

  // Direct copies. Copy k (0..7) of this wave in a stage is stage instruction i = wave + 4k: rows
  // 16i + l/4 of the stage (A rows for i < 16, B rows 16(i-16) + l/4 beyond), lane l filling
  // physical chunk l%4, i.e. logical chunk (l%4) ^ ((l/16) & 3). Each copy gets its own buffer
  // resource over its 16 rows (clamped to the matrix, empty past the tile), so one lane offset
  // serves all eight and rows past the edge read as zero (their outputs are never stored).
  Ctx c;
  c.wave = wave;
  c.wm = wm;
  c.wn = wn;
  c.r32 = r32;
  c.h = h;
  c.nst = nst;
  c.ngroups = ngroups;
  const uint32_t lrow = (uint32_t)(lane >> 2), lchunk = (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
  c.voff = lrow * RB + 16u * lchunk;
#pragma unroll
  for (int k = 0; k < DMA_PER_STAGE; k++) {
    const int i = wave + 4 * k;
    const bool isA = k < 4;
    const int r0 = isA ? 16 * i : 16 * i - BM, rows = isA ? rows_a : rows_b;
    const int nr = max(0, min(16, rows - r0));
    const uint8_t* base = (isA ? p.A + (int64_t)m0 * RB : p.B + (int64_t)n0 * RB) + (int64_t)(nr ? r0 : 0) * RB;
    c.rdata[k] = make_rsrc(base, (uint32_t)nr * RB);
  }
  // Scale copy k of this wave: rows 64i + l with i = wave + 4(k%2) (A rows for even k).
  c.svoff = (uint32_t)lane * nblk;
#pragma unroll
  for (int k = 0; k < F::DMA_PER_GROUP; k++) {
    const int i = wave + 4 * (k & 1);
    const bool isA = (k & 1) == 0;
    const int r0 = isA ? 64 * i : 64 * i - BM, rows = isA ? rows_a : rows_b;
    const int nr = max(0, min(64, rows - r0));
    const uint8_t* base = (isA ? p.SA + (int64_t)m0 * nblk : p.SB + (int64_t)n0 * nblk) + (int64_t)(nr ? r0 : 0) * nblk;
    c.rscale[k] = make_rsrc(base, (uint32_t)nr * nblk);
  }

  v16f acc[T::FB][T::FA];
#pragma unroll
  for (int i = 0; i < T::FB; i++)
#pragma unroll
    for (int j = 0; j < T::FA; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;

  // prologue: scale group 0 and stages 0, 1, 2
  issue_scales<KIND>(c, sgrp, 0);
  for (int t = 0; t < 3 && t < nst; t++) {
    char* slot = t == 0 ? slot0 : (t == 1 ? slot1 : slot2);
#pragma unroll
    for (int k = 0; k < DMA_PER_STAGE; k++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rdata[k], (lds_ptr_t)(slot + (wave + 4 * k) * 1024), 16, c.voff,
                                               ROWB * t, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): prologue copies of this wave
  raw_barrier();
  v8i xa[T::FA], xb[T::FB], ya[T::FA], yb[T::FB];
  Scales<KIND, T> sc;
  RawScales<KIND, T> raw;
  read_raw_scales<KIND, T>(sgrp, raw, 0, wm, wn, r32);
  pack_scales<KIND, T>(raw, sc, 0, h);
  read_raw_scales<KIND, T>(sgrp, raw, 1, wm, wn, r32);
  pack_scales<KIND, T>(raw, sc, 1, h);
#pragma unroll
  for (int j = 0; j < T::FA; j++) xa[j] = read_frag(slot0, row_a<T>(j, wm, r32), h);
#pragma unroll
  for (int i = 0; i < T::FB; i++) xb[i] = read_frag(slot0, row_b<T>(i, wn, r32), h);

  // Stage t uses slot t%4 (t = 8g + s: slot s%4); even stages compute from x*, odd from y*.
  for (int g = 0; g < ngroups; g++) {
    ring_stage<KIND, T, 0>(c, g, sgrp, xa, xb, ya, yb, slot1, slot3, sc, raw, acc);
    ring_stage<KIND, T, 1>(c, g, sgrp, ya, yb, xa, xb, slot2, slot0, sc, raw, acc);
    ring_stage<KIND, T, 2>(c, g, sgrp, xa, xb, ya, yb, slot3, slot1, sc, raw, acc);
    ring_stage<KIND, T, 3>(c, g, sgrp, ya, yb, xa, xb, slot0, slot2, sc, raw, acc);
    ring_stage<KIND, T, 4>(c, g, sgrp, xa, xb, ya, yb, slot1, slot3, sc, raw, acc);
    ring_stage<KIND, T, 5>(c, g, sgrp, ya, yb, xa, xb, slot2, slot0, sc, raw, acc);
    ring_stage<KIND, T, 6>(c, g, sgrp, xa, xb, ya, yb, slot3, slot1, sc, raw, acc);
    ring_stage<KIND, T, 7>(c, g, sgrp, ya, yb, xa, xb, slot0, slot2, sc, raw, acc);
  }

  // The last stages queued copies of stage nst-1 into free slots: let them land, and let every
  // wave finish with the ring, before the slots are reused for the output.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  raw_barrier();

  // Epilogue. The lane holds C[m0 + 32*FA*wm + 32j + r32][n0 + 32*FB*wn + 32i + 8q + 4h + e] in
  // acc[i][j][4q + e]: 8 bytes per row, so storing straight from registers would write each
  // 128-byte line of C in pieces from several instructions. Instead each wave converts to fp16 into
  // its own slot, 32 rows (one A tile) at a time with rows padded by 8 bytes (the 8-byte writes of
  // the 32 rows then fall on distinct banks), and writes the rows back as 16-byte pieces,
  // consecutive lanes along a row.
  char* stage = wave == 0 ? slot0 : (wave == 1 ? slot1 : (wave == 2 ? slot2 : slot3));
  constexpr int WCOLS = 32 * T::FB;            // columns of the wave's block
  constexpr int EROW = 2 * WCOLS + 8;          // staged row pitch, bytes
  constexpr int LPR = WCOLS / 8;               // 16-byte pieces per row
  constexpr int PIECES = 32 * LPR;             // per A tile: a multiple of 64
  static_assert(PIECES % 64 == 0 && 32 * EROW <= SLOT, "epilogue staging");
  const bool rows16 = (p.N & 7) == 0;          // row starts 16-byte aligned
#pragma unroll
  for (int j = 0; j < T::FA; j++) {
#pragma unroll
    for (int i = 0; i < T::FB; i++)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        v4h o;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float v = acc[i][j][4 * q + e];
          o[e] = (_Float16)(p.relu ? fmaxf(v, 0.0f) : v);
        }
        *reinterpret_cast<v4h*>(stage + r32 * EROW + (32 * i + 8 * q + 4 * h) * 2) = o;
      }
#pragma unroll
    for (int s0 = 0; s0 < PIECES; s0 += 64) {
      const int piece = s0 + lane, lr = piece / LPR, cp = piece % LPR;
      const char* src = stage + lr * EROW + 16 * cp;
      const v4h lo = *reinterpret_cast<const v4h*>(src), hi = *reinterpret_cast<const v4h*>(src + 8);
      const int m = m0 + 32 * T::FA * wm + 32 * j + lr, n = n0 + WCOLS * wn + 8 * cp;
      if (m < p.M) {
        _Float16* dst = p.C + (int64_t)m * p.N + n;
        if (n + 8 <= p.N) {
          if (rows16) {
            *reinterpret_cast<v8h*>(dst) = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          } else {
            *reinterpret_cast<v4h*>(dst) = lo;
            *reinterpret_cast<v4h*>(dst + 4) = hi;
          }
        } else if (n + 4 <= p.N) {
          *reinterpret_cast<v4h*>(dst) = lo;
        }
      }
    }
  }
}

}  // namespace

namespace mx {
// MX ring kernels. fp4 = false: E4M3, requires K % 512 == 0; fp4 = true: E2M1, requires
// K % 1024 == 0; both require N % 4 == 0 (checked by the caller). bn = 256 or 224.
int gemm_ring_launch(bool fp4, int bn, const void* A, const void* SA, const void* B, const void* SB, void* C, int M,
                     int N, int K, bool relu, hipStream_t stream) {
  Args a{};
  a.A = (const uint8_t*)A;
  a.SA = (const uint8_t*)SA;
  a.B = (const uint8_t*)B;
  a.SB = (const uint8_t*)SB;
  a.C = (_Float16*)C;
  a.M = M;
  a.N = N;
  a.K = K;
  a.relu = relu ? 1 : 0;
  a.tiles_m = (M + BM - 1) / BM;
  const int tiles = a.tiles_m * ((N + bn - 1) / bn);
  const dim3 grid((unsigned)tiles), block(256);
  if (bn == 224) {
    if (fp4) hipLaunchKernelGGL((gemm_ring_kernel<1, 4>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((gemm_ring_kernel<0, 4>), grid, block, 0, stream, a);
  } else {
    if (fp4) hipLaunchKernelGGL((gemm_ring_kernel<1, 2>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((gemm_ring_kernel<0, 2>), grid, block, 0, stream, a);
  }
  return launch_status();
}
}  // namespace mx
