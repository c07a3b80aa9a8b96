// mxgemm_ring.hip -- MXFP8 (E4M3 x E4M3, E8M0 scales per 32 along K) GEMM with a 4-stage LDS ring.
//
//   C[m,n] = sum_k 2^(SA[m,k/32]-127) A[m,k] * 2^(SB[n,k/32]-127) B[n,k]   (fp32 accumulate, fp16 out)
//
// the block-scaled product of "TensorOps ... notes", sections "Scale planes" and "Kernel-phase
// findings", with the E8M0 scale plane of the WWDC26 session 330 summary; B is K-contiguous.
//
// Why a ring of short stages: a 256x224 tile with 128-byte K stages fills LDS with two stages, so
// each stage's copy has to land within one stage of MFMAs (about 1800 cycles), less than the L2 /
// MALL latency under load. Here a stage is 64 bytes of K, one scaled MFMA 32x32x64 deep:
//  - Tile 256 x 256, 4 waves (one per SIMD), each wave 128 x 128 = 4 x 4 MFMA tiles of 32 x 32.
//  - LDS ring of 4 stages (4 separate arrays, so the compiler can tell a fragment read of one
//    stage from the direct copies filling another): 256 + 256 rows x 64 bytes per stage. Copies for
//    stage t+3 are queued while stage t computes, three stages (about 3000 cycles) ahead.
//  - 64-byte rows hold four 16-byte chunks, stored at chunk ^ ((row >> 2) & 3): a 16-lane quarter of
//    a fragment read (16 rows, one chunk) then covers all 64 banks once.
//  - Direct global->LDS copies (16 bytes per lane): instruction i of a stage fills rows
//    16i..16i+15; lane l fills physical chunk l%4 of row 16i + l/4.
//  - E8M0 scales for 8 stages (16 bytes per row) are copied once per group into the scale array
//    (after every wave has read the previous group's); each lane packs its own K-block's bytes so that byte s%4 of dword s/4 is its scale for
//    stage s of the group (op_sel picks the byte).
//  - Fragments of stage t+1 are read from LDS while the MFMAs of stage t run; one barrier per
//    stage, after this wave's copies of stage t+1 have landed (vmcnt), publishes stage t+1 and
//    frees the slot of stage t-1.
// Operand layout of v_mfma_scale_f32_32x32x64_f8f6f4 (measured): lane l feeds row l%32 and K bytes
// 16h..16h+15 and 32+16h..32+16h+15 (h = l/32) and supplies the scale of (row l%32, K-block h);
// output element e of lane l is row 8(e/4) + 4h + e%4 of the first operand and column l%32 of the
// second. B is the first operand, so each lane ends with 4 consecutive n of one row m.
#include <type_traits>

#include "common.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int BM = 256, BN = 256;       // tile
constexpr int ROWB = 64;                // K bytes per stage
constexpr int ROWS = BM + BN;           // LDS rows per stage (A then B)
constexpr int SLOT = ROWS * ROWB;       // 32 KB
constexpr int SGRP = ROWS * 16;         // 8 KB: scales of 8 stages
constexpr int GROUP = 8;                // stages per scale group
constexpr int DMA_PER_STAGE = SLOT / 1024 / 4;  // direct copies per wave per stage (8)
constexpr int DMA_PER_GROUP = SGRP / 1024 / 4;  // direct copies per wave per scale group (2)

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
};

struct Scales {
  uint32_t a[4][2], b[4][2];  // per lane: byte S8%4 of dword S8/4 = this lane's scale for stage S8 of the group
};

MX_DEV int phys_off(int row, int chunk) { return row * ROWB + ((chunk ^ ((row >> 2) & 3)) << 4); }

MX_DEV v4i lds16(const char* base, int off) { return *reinterpret_cast<const v4i*>(base + off); }

// The lane's 16 scale bytes of a row hold (stage s, block b) at byte 2s + b. Half d (bytes 8d..8d+7,
// stages 4d..4d+3) becomes dword d of the lane's packed scales, keeping its own block h: bytes h,
// 2+h, 4+h, 6+h. Stages 0-3 of a group use dword 0 and stages 4-7 dword 1, so the next group's
// half 0 is read during stage 4 and packed at the end of stage 6, and its half 1 is read after
// the last MFMA of stage 7 and packed at the end of the next group's stage 2: the reads have a
// stage or more to land before anything waits for them. The packed value of stage 2 is unchanged
// in group 0, whose halves the prologue packs.
typedef int v2i __attribute__((ext_vector_type(2)));
struct RawScales {
  v2i a[4], b[4];
};

MX_DEV void read_raw_scales(const char* sg, RawScales& r, int d, int wm, int wn, int r32) {
#pragma unroll
  for (int j = 0; j < 4; j++) r.a[j] = *reinterpret_cast<const v2i*>(sg + (128 * wm + 32 * j + r32) * 16 + 8 * d);
#pragma unroll
  for (int i = 0; i < 4; i++)
    r.b[i] = *reinterpret_cast<const v2i*>(sg + (BM + 128 * wn + 32 * i + r32) * 16 + 8 * d);
}

MX_DEV void pack_scales(const RawScales& r, Scales& s, int d, int h) {
  const uint32_t sel = h ? 0x07050301u : 0x06040200u;
#pragma unroll
  for (int j = 0; j < 4; j++) s.a[j][d] = __builtin_amdgcn_perm((uint32_t)r.a[j][1], (uint32_t)r.a[j][0], sel);
#pragma unroll
  for (int i = 0; i < 4; i++) s.b[i][d] = __builtin_amdgcn_perm((uint32_t)r.b[i][1], (uint32_t)r.b[i][0], sel);
}

// B fragment i of one stage (rows 256 + 128*wn + 32i + l%32) and A fragment j (rows 128*wm + 32j).
MX_DEV v8i read_b(const char* slot, int i, int wn, int r32, int h) {
  const int row = BM + 128 * wn + 32 * i + r32;
  return __builtin_shufflevector(lds16(slot, phys_off(row, h)), lds16(slot, phys_off(row, 2 + h)), 0, 1, 2, 3, 4, 5,
                                 6, 7);
}
MX_DEV v8i read_a(const char* slot, int j, int wm, int r32, int h) {
  const int row = 128 * wm + 32 * j + r32;
  return __builtin_shufflevector(lds16(slot, phys_off(row, h)), lds16(slot, phys_off(row, 2 + h)), 0, 1, 2, 3, 4, 5,
                                 6, 7);
}

// Per-workgroup constants of the main loop.
struct Ctx {
  rsrc_t rdata[DMA_PER_STAGE];
  rsrc_t rscale[DMA_PER_GROUP];
  uint32_t voff, svoff;
  int wave, wm, wn, r32, h, nst, ngroups;
};

MX_DEV void issue_scales(const Ctx& c, char* sg, int g) {
#pragma unroll
  for (int k = 0; k < DMA_PER_GROUP; k++)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rscale[k], (lds_ptr_t)(sg + (c.wave + 4 * k) * 1024), 16, c.svoff,
                                             16 * g, 0, 0);
}

// One stage t = 8g + S8: slot t%4 holds stage t (its fragments already in ca/cb). Before the
// barrier this wave's copies of stage t+1 must have landed; after it, slot (t+3)%4 (stage t-1,
// read during stage t-2) is free and stage t+1 is readable by every wave. The MFMAs go B tile by B
// tile; after each tile come two copies of stage t+3 and two of the next stage's fragments, into
// the other register set (dead during this stage): the A fragments first, as the next stage's first
// B tile needs all four, then the B fragments in the order their tiles come.
// The next-stage reads are unconditional (after the last stage they fetch unused bytes): a
// conditional overwrite would keep the old contents alive through the stage.
template <int S8>
MX_DEV void ring_stage(const Ctx& c, int g, char* sgrp, const v8i (&ca)[4], const v8i (&cb)[4],
                       v8i (&na)[4], v8i (&nb)[4], const char* slot_nxt, char* slot_fill, Scales& sc,
                       RawScales& raw, v16f (&acc)[4][4]) {
  constexpr int D = S8 / 4, OP = S8 % 4;
  const int t = GROUP * g + S8;
  // Copies queued after this wave's copies of stage t+1 (issued at stage t-2): those of stage t+2
  // (at stage t-1) and, at S8 == 3, the scale group issued at S8 == 2 ahead of them. From S8 == 4
  // on, the next group's scales are visible.
  wait_vm_n(S8 == 3 ? DMA_PER_STAGE + DMA_PER_GROUP : DMA_PER_STAGE);
  raw_barrier();
  // The scale array still holds half 1 of group g, read at the end of stage 7 of group g-1. Every
  // wave has waited for those reads before stage 1's MFMAs (they precede the fragment reads of
  // stage 0 in the wave's LDS queue), so past stage 2's barrier the array is free.
  if (S8 == 2) issue_scales(c, sgrp, min(g + 1, c.ngroups - 1));
  const uint32_t fill_off = ROWB * min(t + 3, c.nst - 1);
#pragma unroll
  for (int i = 0; i < 4; i++) {
#pragma unroll
    for (int j = 0; j < 4; j++)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cb[i], ca[j], acc[i][j], 0, 0, OP, sc.b[i][D], OP,
                                                                   sc.a[j][D]);
#pragma unroll
    for (int k = 2 * i; k < 2 * i + 2; k++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rdata[k], (lds_ptr_t)(slot_fill + (c.wave + 4 * k) * 1024), 16,
                                               c.voff, fill_off, 0, 0);
    if (i < 2) {
      na[2 * i] = read_a(slot_nxt, 2 * i, c.wm, c.r32, c.h);
      na[2 * i + 1] = read_a(slot_nxt, 2 * i + 1, c.wm, c.r32, c.h);
    } else {
      nb[2 * i - 4] = read_b(slot_nxt, 2 * i - 4, c.wn, c.r32, c.h);
      nb[2 * i - 3] = read_b(slot_nxt, 2 * i - 3, c.wn, c.r32, c.h);
    }
    if (S8 == 4 && i == 1) read_raw_scales(sgrp, raw, 0, c.wm, c.wn, c.r32);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (S8 == 2) pack_scales(raw, sc, 1, c.h);
  if (S8 == 6) pack_scales(raw, sc, 0, c.h);
  if (S8 == GROUP - 1) read_raw_scales(sgrp, raw, 1, c.wm, c.wn, c.r32);
}

__global__ __launch_bounds__(256, 1) void gemm_ring_kernel(Args p) {
  __shared__ __attribute__((aligned(16))) char slot0[SLOT];
  __shared__ __attribute__((aligned(16))) char slot1[SLOT];
  __shared__ __attribute__((aligned(16))) char slot2[SLOT];
  __shared__ __attribute__((aligned(16))) char slot3[SLOT];
  __shared__ __attribute__((aligned(16))) char sgrp[SGRP];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int r32 = lane & 31, h = lane >> 5;

  int bid = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);  // each XCD takes a contiguous tile range
  const int tm = bid % p.tiles_m, tn = bid / p.tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int rows_a = min(BM, p.M - m0), rows_b = min(BN, p.N - n0);
  const uint32_t K = (uint32_t)p.K, nblk = K / 32;
  const int nst = p.K / ROWB, ngroups = nst / GROUP;

  // Direct copies. Copy k (0..7) of this wave in a stage is stage instruction i = wave + 4k: rows
  // 16i + l/4 of the stage (A rows for k < 4, B rows 16(i-16) + l/4 for k >= 4), lane l filling
  // physical chunk l%4, i.e. logical chunk (l%4) ^ ((l/16) & 3). Each copy gets its own buffer
  // resource over its 16 rows (clamped to the matrix), so one lane offset serves all eight and rows
  // past the edge fall outside the resource and read as zero (their outputs are never stored).
  Ctx c;
  c.wave = wave;
  c.wm = wm;
  c.wn = wn;
  c.r32 = r32;
  c.h = h;
  c.nst = nst;
  c.ngroups = ngroups;
  const uint32_t lrow = (uint32_t)(lane >> 2), lchunk = (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
  c.voff = lrow * K + 16u * lchunk;
#pragma unroll
  for (int k = 0; k < DMA_PER_STAGE; k++) {
    const int i = wave + 4 * k;
    const bool isA = k < 4;
    const int r0 = isA ? 16 * i : 16 * i - BM, rows = isA ? rows_a : rows_b;
    const int nr = max(0, min(16, rows - r0));
    const uint8_t* base = (isA ? p.A + (int64_t)m0 * K : p.B + (int64_t)n0 * K) + (int64_t)(nr ? r0 : 0) * K;
    c.rdata[k] = make_rsrc(base, (uint32_t)nr * K);
  }
  // Scale copy k (0, 1) of this wave: instruction i = wave + 4k, rows 64i + l (A for k == 0).
  c.svoff = (uint32_t)lane * nblk;
#pragma unroll
  for (int k = 0; k < DMA_PER_GROUP; k++) {
    const int i = wave + 4 * k;
    const bool isA = k == 0;
    const int r0 = isA ? 64 * i : 64 * i - BM, rows = isA ? rows_a : rows_b;
    const int nr = max(0, min(64, rows - r0));
    const uint8_t* base = (isA ? p.SA + (int64_t)m0 * nblk : p.SB + (int64_t)n0 * nblk) + (int64_t)(nr ? r0 : 0) * nblk;
    c.rscale[k] = make_rsrc(base, (uint32_t)nr * nblk);
  }

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;

  // prologue: scale group 0 and stages 0, 1, 2
  issue_scales(c, sgrp, 0);
  for (int t = 0; t < 3 && t < nst; t++) {
    char* slot = t == 0 ? slot0 : (t == 1 ? slot1 : slot2);
#pragma unroll
    for (int k = 0; k < DMA_PER_STAGE; k++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rdata[k], (lds_ptr_t)(slot + (wave + 4 * k) * 1024), 16, c.voff,
                                               ROWB * t, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): prologue copies of this wave
  raw_barrier();
  v8i xa[4], xb[4], ya[4], yb[4];
  Scales sc;
  RawScales raw;
  read_raw_scales(sgrp, raw, 0, wm, wn, r32);
  pack_scales(raw, sc, 0, h);
  read_raw_scales(sgrp, raw, 1, wm, wn, r32);
  pack_scales(raw, sc, 1, h);
#pragma unroll
  for (int j = 0; j < 4; j++) xa[j] = read_a(slot0, j, wm, r32, h);
#pragma unroll
  for (int i = 0; i < 4; i++) xb[i] = read_b(slot0, i, wn, r32, h);

  // Stage t uses slot t%4 (t = 8g + s: slot s%4); even stages compute from x*, odd from y*.
  for (int g = 0; g < ngroups; g++) {
    ring_stage<0>(c, g, sgrp, xa, xb, ya, yb, slot1, slot3, sc, raw, acc);
    ring_stage<1>(c, g, sgrp, ya, yb, xa, xb, slot2, slot0, sc, raw, acc);
    ring_stage<2>(c, g, sgrp, xa, xb, ya, yb, slot3, slot1, sc, raw, acc);
    ring_stage<3>(c, g, sgrp, ya, yb, xa, xb, slot0, slot2, sc, raw, acc);
    ring_stage<4>(c, g, sgrp, xa, xb, ya, yb, slot1, slot3, sc, raw, acc);
    ring_stage<5>(c, g, sgrp, ya, yb, xa, xb, slot2, slot0, sc, raw, acc);
    ring_stage<6>(c, g, sgrp, xa, xb, ya, yb, slot3, slot1, sc, raw, acc);
    ring_stage<7>(c, g, sgrp, ya, yb, xa, xb, slot0, slot2, sc, raw, acc);
  }

  // The last stages queued copies of stage nst-1 into free slots: let them land, and let every
  // wave finish with the ring, before the slots are reused for the output.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  raw_barrier();

  // Epilogue. The lane holds C[m0 + 128wm + 32j + r32][n0 + 128wn + 32i + 8q + 4h + e] in
  // acc[i][j][4q + e]: 8 bytes per row, so storing straight from registers would write each
  // 128-byte line of C in eight pieces from eight instructions. Instead each wave converts to fp16
  // into its own slot, 64 rows at a time (rows padded to 264 bytes: the 8-byte writes of 32 rows
  // then fall on distinct banks), and writes the rows back 16 bytes per lane, 256 contiguous bytes
  // per row.
  char* stage = wave == 0 ? slot0 : (wave == 1 ? slot1 : (wave == 2 ? slot2 : slot3));
  constexpr int EROW = 264;
#pragma unroll
  for (int half = 0; half < 2; half++) {
#pragma unroll
    for (int jj = 0; jj < 2; jj++)
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          v4h o;
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const float v = acc[i][2 * half + jj][4 * q + e];
            o[e] = (_Float16)v;
          }
          *reinterpret_cast<v4h*>(stage + (32 * jj + r32) * EROW + (32 * i + 8 * q + 4 * h) * 2) = o;
        }
    // 64 rows x 256 bytes: instruction s covers rows 4s..4s+3, lane l row 4s + l/16, bytes 16(l%16)
    const int cl = lane & 15, n = n0 + 128 * wn + 8 * cl;
#pragma unroll
    for (int s4 = 0; s4 < 16; s4++) {
      const int lr = 4 * s4 + (lane >> 4);
      const int m = m0 + 128 * wm + 64 * half + lr;
      typedef _Float16 v8h __attribute__((ext_vector_type(8)));
      const char* src = stage + lr * EROW + 16 * cl;
      const v4h lo = *reinterpret_cast<const v4h*>(src), hi = *reinterpret_cast<const v4h*>(src + 8);
      if (m < p.M) {
        _Float16* dst = p.C + (int64_t)m * p.N + n;
        if (n + 8 <= p.N) {
          if ((p.N & 7) == 0) {  // rows start 16-byte aligned
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
// MXFP8 ring kernel: requires K % 512 == 0 and N % 4 == 0 (checked by the caller).
int gemm_ring_launch(const void* A, const void* SA, const void* B, const void* SB, void* C, int M, int N, int K,
                     hipStream_t stream) {
  Args a{};
  a.A = (const uint8_t*)A;
  a.SA = (const uint8_t*)SA;
  a.B = (const uint8_t*)B;
  a.SB = (const uint8_t*)SB;
  a.C = (_Float16*)C;
  a.M = M;
  a.N = N;
  a.K = K;
  a.tiles_m = (M + BM - 1) / BM;
  const int tiles = a.tiles_m * ((N + BN - 1) / BN);
  hipLaunchKernelGGL(gemm_ring_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, a);
  return launch_status();
}
}  // namespace mx
