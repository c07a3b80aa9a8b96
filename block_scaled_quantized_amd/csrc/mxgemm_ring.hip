// mxgemm_ring.hip -- MX GEMMs (E8M0 scales per 32 along K) on two kernels: a 4-stage LDS ring of
// 64-byte stage rows (every MX pair, and fp16) and, further below, an 8-wave ping-pong kernel of
// 128-byte stage rows (the byte formats E4M3 / E5M2, E2M1 x E2M1 and the FP6 pairs, K % 1024 == 0;
// fp16 x fp16, K % 512 == 0).
//
//   C[m,n] = sum_k 2^(SA[m,k/32]-127) A[m,k] * 2^(SB[n,k/32]-127) B[n,k]   (fp32 accumulate, fp16 out)
//
// the block-scaled product of "TensorOps ... notes", sections "Scale planes" and "Kernel-phase
// findings", with the E8M0 scale plane of the WWDC26 session 330 summary; B is K-contiguous.
//
// Why a ring of short stages: a 256x224 tile with 128-byte K stages fills LDS with two stages, so
// each stage's copy has to land within one stage of MFMAs (about 1800 cycles), less than the L2 /
// MALL latency under load. Here a stage is one scaled MFMA 32x32x64 deep (64 bytes of an E4M3 row,
// 32 of an E2M1 row), two for E2M1 x E2M1 (64 bytes of each row).
//  - Tile 256 x 256 with 4 waves (one per SIMD) of 128 x 128 = 4 x 4 MFMA tiles of 32 x 32, or
//    256 x 224 with 4 waves of 64 x 224 = 2 x 7 MFMA tiles (224 = 7 x 32 does not split in two:
//    the 256 x 224 tile exists so that N = 14336 gives 64 column tiles, a whole number of rounds
//    on 256 CUs at M = 2048).
//  - LDS ring of 4 stages (4 separate arrays, so the compiler can tell a fragment read of one
//    stage from the direct copies filling another): up to 256 + 256 rows x 64 bytes per stage.
//    Copies for stage t+3 are queued while stage t computes, three stages ahead.
//  - 64-byte rows hold four 16-byte chunks, stored at chunk ^ ((row >> 2) & 3) (32-byte rows: two,
//    at chunk ^ ((row >> 3) & 1)): a 16-lane quarter of a fragment read (16 rows, one chunk) then
//    covers all 64 banks once.
//  - Direct global->LDS copies (16 bytes per lane): instruction i of a stage fills 1 KB, rows
//    16i..16i+15 of 64 bytes (lane l: physical chunk l%4 of row 16i + l/4) or 32 rows of 32
//    bytes. Each wave issues 8 per stage (6 for a mixed pair);
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
constexpr int ROWB = 64;                // bytes per operand row per stage, at most
constexpr int SLOT = 512 * ROWB;        // 32 KB: room for 256 + 256 rows
constexpr int GROUP = 8;                // stages per scale group
constexpr int MAX_DPS = 8;              // direct copies per wave per stage, at most

// Tile shapes. WAVES_M waves along M (the rest along N); each wave holds FA x FB MFMA tiles of
// 32 x 32 (FA along M, FB along N). 256 x 256 and 256 x 192 with 2 x 2 waves, 256 x 224 with 4 x 1.
template <int WAVES_M_, int BN_>
struct RingTile {
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = 4 / WAVES_M;
  static constexpr int BN = BN_;
  static constexpr int FA = BM / 32 / WAVES_M, FB = BN / 32 / WAVES_N;
  static constexpr int F = FA + FB;  // fragments read per stage per wave
  static_assert((WAVES_M == 2 && (BN == 256 || BN == 192)) || (WAVES_M == 4 && BN == 224), "tile");
};

// Per-format constants. KIND 0: E4M3 x E4M3, 1: E2M1 x E2M1, 2: E4M3 A x E2M1 B, 3: E2M1 A x E4M3 B,
// 4: fp16 x fp16 (no scales), 5: FP6 x FP6 (E2M3 / E3M2: a stage row is 48 bytes in memory, copied
// as four 12-byte pieces, one per 16-byte LDS chunk: a 12-byte direct copy writes lane i at 16 i,
// measured).
// A stage is one MFMA K-step of 64 elements (2 scale blocks), or for E2M1 x E2M1 two K-steps of
// 64 (128 elements, 4 blocks) so that its rows are 64 bytes too. An operand's stage row is 64 bytes,
// or 32 for the E2M1 side of a mixed pair. A group of 8 stages holds 16 or 32 scale bytes per row,
// and each lane keeps 8 or 16 of them (its own K-block h of every K-step), 2 or 4 dwords.
// fp16: a stage is 32 K-elements, two K-steps of the 32x32x16 fp16 MFMA; A rows are 64 bytes as
// above, and B (K x N, N-contiguous) is staged as 32 K-rows of 512 bytes (256 columns), read with
// transposing LDS loads.
template <int KIND>
struct RingFmt {
  // (enumerators rather than static data members: the host pass of hipcc sees these in device-only
  // templates, where it mishandles static constexpr members)
  enum : int {
    F16 = KIND == 4,                                   // fp16 x fp16: no scale plane
    F6 = KIND == 5,                                    // FP6 x FP6: 48-byte stage rows in memory
    CPY = F6 ? 12 : 16,                                // bytes per lane of a stage copy
    CPYB = 1024,                                       // LDS bytes of one copy instruction
    A4 = KIND == 1 || KIND == 3, B4 = KIND == 1 || KIND == 2,  // E2M1 operands
    FP4 = KIND == 1,                                   // both E2M1: two K-steps per stage, two scale planes
    KSTEPS = FP4 || F16 ? 2 : 1,                       // MFMA K-steps per stage
    ELEMS = F16 ? 32 : 64 * KSTEPS,                    // K elements per stage
    SRB_A = A4 && !FP4 ? 32 : 64, SRB_B = B4 && !FP4 ? 32 : 64,  // LDS bytes per stage row (fp16 B: per 16 columns)
    GSB_A = F6 ? 48 : SRB_A, GSB_B = F6 ? 48 : SRB_B,  // bytes per stage row in memory
    NI_A = BM * SRB_A / CPYB,                          // copy instructions per stage for A (16 / 8)
    NI_B = 256 * SRB_B / CPYB,                         // ... and for B (room for 256 rows / columns)
    DPS = (NI_A + NI_B) / 4,                           // copies per wave per stage (8 or 6)
    CBSZ = B4 ? 4 : 0, BLGP = A4 ? 4 : 0,              // MFMA formats of the B and A operands
    SGRP = F16 ? 16 : 512 * 16 * KSTEPS,               // scale array: 8 / 16 KB (fp16: unused)
    SDW = 2 * KSTEPS,                                  // packed scale dwords per row per lane
    DMA_PER_GROUP = F16 ? 0 : SGRP / 1024 / 4          // scale copies per wave per group (2 / 4)
  };
  static_assert(NI_A % 4 == 0 && NI_B % 4 == 0 && DPS <= MAX_DPS, "copies");
};

// MFMA format codes of the two operands (the instruction's cbsz for its first operand, our B, and
// blgp for the second, our A): 4 for E2M1; for a byte operand 0 (E4M3) or 1 (E5M2) as given by
// F8A / F8B. E5M2 has E4M3's storage and layout, so only these codes change.
template <int KIND, int F8A, int F8B>
struct RingMfma {
  enum : int { CBSZ = RingFmt<KIND>::B4 ? 4 : F8B, BLGP = RingFmt<KIND>::A4 ? 4 : F8A };
};

// Copies of a stage for a tile width: NI_A for A, then enough 1 KB copies for the tile's B rows,
// rounded up so that the 4 waves issue the same number (the extra ones fill unused slot bytes with
// zeros from an empty resource): DPS per wave.
template <int KIND, class T>
struct RingCopies {
  enum : int {
    NI_A = RingFmt<KIND>::NI_A,
    NI_B0 = (T::BN * RingFmt<KIND>::SRB_B + RingFmt<KIND>::CPYB - 1) / RingFmt<KIND>::CPYB,
    NI_B = (NI_A + NI_B0 + 3) / 4 * 4 - NI_A,
    DPS = (NI_A + NI_B) / 4
  };
  static_assert(DPS <= MAX_DPS && (!RingFmt<KIND>::F16 || T::BN == 256), "copies");
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
  int M, N, K, tiles_m, tiles_n;
  int relu;  // epilogue: C = max(C, 0) (IEEE maxNum: NaN gives 0)
};

// Per lane: byte u%4 of dword u/4 is the lane's scale for MFMA K-step u of the group (u = stage for
// E4M3, 2*stage + k for K-step k of a stage for E2M1).
template <int KIND, class T>
struct Scales {
  uint32_t a[T::FA][RingFmt<KIND>::SDW], b[T::FB][RingFmt<KIND>::SDW];
};

// Byte offset of 16-byte chunk `chunk` of row `row` within an operand's region of a slot. 64-byte
// rows store chunk c at c ^ ((row >> 2) & 3) and 32-byte rows at c ^ ((row >> 3) & 1): the 16 rows
// of a quarter-wave fragment read then cover all 64 banks once.
template <int SRB>
MX_DEV int phys_off(int row, int chunk) {
  if constexpr (SRB == 64) return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4);
  else return row * 32 + ((chunk ^ ((row >> 3) & 1)) << 4);
}

MX_DEV v4i lds16(const char* base, int off) { return *reinterpret_cast<const v4i*>(base + off); }

// Scale layout in LDS. E4M3: row r's 16 bytes of the group at r*16, (stage s, block b) at byte
// 2s + b. E2M1: two planes of 8 KB (stages 0-3, 4-7), row r's 16 bytes of plane d at d*8192 + r*16,
// (stage s, K-step k, block b) at byte 4(s%4) + 2k + b. Half d of a row covers stages 4d..4d+3
// and becomes dwords d*KSTEPS.. of the lane's packed scales, keeping its own block h: from each 8
// source bytes, bytes h, 2+h, 4+h, 6+h. Stages 0-3 of a group use the dwords of half 0 and stages
// 4-7 those of half 1, so both halves of the next group are read during stage 4 (into separate
// registers); half 0 is packed at the end of stage 6 and half 1 at the end of the next group's
// stage 2: the reads have a stage or more to land before anything waits for them. (An LDS read
// placed after the last stage of a group lands at the loop head, where the compiler makes it wait
// for every direct copy in flight.) The packed value of stage 2 is unchanged in group 0, whose
// halves the prologue packs.
template <int KIND>
struct RawT {
  typedef int type __attribute__((ext_vector_type(2 * RingFmt<KIND>::KSTEPS)));
};

template <int KIND, class T>
struct RawScales {
  typename RawT<KIND>::type a[T::FA], b[T::FB];
};

// Rows of the wave's fragments within their operand: A fragment j is row 32*FA*wm + 32j + l%32,
// B fragment i is row 32*FB*wn + 32i + l%32. The scale array numbers A rows 0..255 and B rows from
// 256 (BM) on.
template <class T>
MX_DEV int row_a(int j, int wm, int r32) { return 32 * T::FA * wm + 32 * j + r32; }
template <class T>
MX_DEV int row_b(int i, int wn, int r32) { return 32 * T::FB * wn + 32 * i + r32; }

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
  for (int i = 0; i < T::FB; i++) r.b[i] = raw_at<KIND>(sg, BM + row_b<T>(i, wn, r32), d);
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

// A fragment of one stage. 64-byte rows: chunks h and 2+h, i.e. the lane's K bytes of the E4M3
// MFMA, or its 16 bytes (K-block h) of E2M1 K-steps 0 and 1 in the low and high halves. 32-byte rows
// (the E2M1 side of a mixed pair): chunk h, the lane's 16 bytes, in the low half.
// FP6 fragment: the lane's 32 elements (K-block h) are the 24 bytes 24h.. of its 48-byte row, i.e.
// pieces 2h and 2h+1 (12 bytes each) of the row's four 16-byte chunks.
typedef int v3i __attribute__((ext_vector_type(3)));
MX_DEV v8i read_frag6(const char* region, int row, int h) {
  const v3i lo = *reinterpret_cast<const v3i*>(region + phys_off<64>(row, 2 * h));
  const v3i hi = *reinterpret_cast<const v3i*>(region + phys_off<64>(row, 2 * h + 1));
  const v4i a = __builtin_shufflevector(lo, lo, 0, 1, 2, -1), b = __builtin_shufflevector(hi, hi, 0, 1, 2, -1);
  return __builtin_shufflevector(a, b, 0, 1, 2, 4, 5, 6, -1, -1);
}

template <int SRB>
MX_DEV v8i read_frag(const char* region, int row, int h) {
  if constexpr (SRB == 64)
    return __builtin_shufflevector(lds16(region, phys_off<64>(row, h)), lds16(region, phys_off<64>(row, 2 + h)), 0, 1,
                                   2, 3, 4, 5, 6, 7);
  else {
    const v4i x = lds16(region, phys_off<32>(row, h));
    return __builtin_shufflevector(x, x, 0, 1, 2, 3, -1, -1, -1, -1);
  }
}

// fp16 B fragment of one stage from the staged K x 256 block (32 rows of 512 bytes; 16-byte chunk c
// of row k stored at chunk c ^ 4(k & 3)). ds_read_b64_tr_b16 (measured on gfx950): within each
// 16-lane group, output lane j element r is element j%4 of the 8 bytes that lane j/4 + 4r
// addressed. With lane i of a group addressing row i/4 (plus the group's K offset), columns
// 4(i%4)..+3 of the group's 16, lane j receives column j at 4 consecutive K. Lane l (h = l/32) thus
// gets column l%32 of the B tile at K = 16s + 8h + 0..7 for K-step s: the same K as its A fragment
// (chunk 2s + h of its A row). `off` is the lane's byte offset for K-step 0, first half; the other
// three reads are 4 and 16 rows on. A half-wave reads 4 rows x 64 bytes, whose chunks the swizzle
// puts on all 64 banks once.
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;
MX_DEV v2i lds_tr8(const char* p) {
  return __builtin_bit_cast(v2i, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(
                                     (__attribute__((address_space(3))) char*)p)));
}
MX_DEV v8i read_frag_bt(const char* region, uint32_t off) {
  const v2i r0 = lds_tr8(region + off), r1 = lds_tr8(region + off + 4 * 512);
  const v2i r2 = lds_tr8(region + off + 16 * 512), r3 = lds_tr8(region + off + 20 * 512);
  const v4i lo = __builtin_shufflevector(r0, r1, 0, 1, 2, 3), hi = __builtin_shufflevector(r2, r3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Per-workgroup constants of the main loop (rscale: the first DMA_PER_GROUP of the format are set).
struct Ctx {
  rsrc_t rdata[MAX_DPS];
  rsrc_t rscale[4];
  uint32_t voff_a, voff_b, svoff;  // lane offsets of the A and B stage copies and of the scale copies
  uint32_t bstage;                 // fp16: bytes between the B rows of consecutive stages (32 rows)
  uint32_t bt_off[4];              // fp16: the lane's B fragment offsets (read_frag_bt), per B tile
  int wave, wm, wn, r32, h, nst, ngroups;
};

// Wave-uniform offset of a stage copy: along the row for A and MX B, 32 rows down for fp16 B.
template <int KIND>
MX_DEV uint32_t stage_soff(const Ctx& c, bool qa, uint32_t stage) {
  using F = RingFmt<KIND>;
  uint32_t step_b;
  if constexpr (F::F16) step_b = c.bstage;
  else step_b = (uint32_t)F::GSB_B;
  return (qa ? (uint32_t)F::GSB_A : step_b) * stage;
}

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

// Stage copy q of this wave (copy q is an A copy when q < NI_A/4) into the slot being filled.
template <int KIND>
MX_DEV void stage_copy(const Ctx& c, int q, char* slot_fill, uint32_t fill_stage) {
  using F = RingFmt<KIND>;
  // (offsets computed into locals first: the host pass of hipcc drops the kernel, silently, when
  // these builtin arguments are written as conditional expressions of the format constants)
  const bool qa = q < F::NI_A / 4;
  const uint32_t vo = qa ? c.voff_a : c.voff_b;
  const uint32_t so = stage_soff<KIND>(c, qa, fill_stage);
  if constexpr (F::F6)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rdata[q], (lds_ptr_t)(slot_fill + (c.wave + 4 * q) * 1024), 12, vo, so,
                                             0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rdata[q], (lds_ptr_t)(slot_fill + (c.wave + 4 * q) * 1024), 16, vo, so,
                                             0, 0);
}

// Fragment f of the next stage (A0.., then B0..) from its slot into the other register set.
template <int KIND, class T>
MX_DEV void next_frag(const Ctx& c, int f, const char* slot_nxt, v8i (&na)[T::FA], v8i (&nb)[T::FB]) {
  using F = RingFmt<KIND>;
  if constexpr (F::F6) {
    if (f < T::FA) na[f] = read_frag6(slot_nxt, row_a<T>(f, c.wm, c.r32), c.h);
    else nb[f - T::FA] = read_frag6(slot_nxt + BM * F::SRB_A, row_b<T>(f - T::FA, c.wn, c.r32), c.h);
  } else if (f < T::FA) na[f] = read_frag<F::SRB_A>(slot_nxt, row_a<T>(f, c.wm, c.r32), c.h);
  else if constexpr (F::F16) nb[f - T::FA] = read_frag_bt(slot_nxt + BM * F::SRB_A, c.bt_off[f - T::FA]);
  else nb[f - T::FA] = read_frag<F::SRB_B>(slot_nxt + BM * F::SRB_A, row_b<T>(f - T::FA, c.wn, c.r32), c.h);
}

// One stage t = 8g + S8: slot t%4 holds stage t (its fragments already in ca/cb). Before the
// barrier this wave's copies of stage t+1 must have landed; after it, slot (t+3)%4 (stage t-1,
// read during stage t-2) is free and stage t+1 is readable by every wave. The MFMAs go B tile by B
// tile; after each tile come its share of the 8 copies of stage t+3 and of the next stage's
// fragments, read into the other register set (dead during this stage): the A fragments first, as
// the next stage's first B tile needs all of them, then the B fragments in the order their tiles
// come. The next-stage reads are unconditional (after the last stage they fetch unused bytes): a
// conditional overwrite would keep the old contents alive through the stage.
template <int KIND, class T, int S8, int F8A, int F8B>
MX_DEV void ring_stage(const Ctx& c, int g, char* sgrp, const v8i (&ca)[T::FA], const v8i (&cb)[T::FB],
                       v8i (&na)[T::FA], v8i (&nb)[T::FB], const char* slot_nxt, char* slot_fill,
                       Scales<KIND, T>& sc, RawScales<KIND, T>& raw, RawScales<KIND, T>& raw1,
                       v16f (&acc)[T::FB][T::FA]) {
  using F = RingFmt<KIND>;
  using CP = RingCopies<KIND, T>;
  using MF = RingMfma<KIND, F8A, F8B>;
  const int t = GROUP * g + S8;
  // Copies queued after this wave's copies of stage t+1 (issued at stage t-2): those of stage t+2
  // (at stage t-1) and, at S8 == 3, the scale group issued at S8 == 2 ahead of them. From S8 == 4
  // on, the next group's scales are visible.
  wait_vm_n(S8 == 3 ? CP::DPS + F::DMA_PER_GROUP : CP::DPS);
  raw_barrier();
  // The scale array holds group g, both halves read during stage 4 of group g-1. Every wave has
  // waited for those reads before stage 5's MFMAs (they precede the fragment reads of stage 5 in
  // the wave's LDS queue), so past stage 2's barrier the array is free.
  if constexpr (!F::F16)
    if (S8 == 2) issue_scales<KIND>(c, sgrp, min(g + 1, c.ngroups - 1));
  const uint32_t fill_stage = (uint32_t)min(t + 3, c.nst - 1);
#pragma unroll
  for (int i = 0; i < T::FB; i++) {
#pragma unroll
    for (int k = 0; k < F::KSTEPS; k++) {
      constexpr int U0 = F::KSTEPS * S8;  // first K-step of the stage within the group
#pragma unroll
      for (int j = 0; j < T::FA; j++) {
        if constexpr (F::F16) {
          const v8h bk = __builtin_bit_cast(v8h, k ? __builtin_shufflevector(cb[i], cb[i], 4, 5, 6, 7)
                                                   : __builtin_shufflevector(cb[i], cb[i], 0, 1, 2, 3));
          const v8h ak = __builtin_bit_cast(v8h, k ? __builtin_shufflevector(ca[j], ca[j], 4, 5, 6, 7)
                                                   : __builtin_shufflevector(ca[j], ca[j], 0, 1, 2, 3));
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bk, ak, acc[i][j], 0, 0, 0);
        } else if constexpr (F::FP4) {
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
          // E4M3 x E4M3 or a mixed pair: one K-step; the E2M1 side's fragment is its low half
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cb[i], ca[j], acc[i][j], MF::CBSZ, MF::BLGP, U0 % 4,
                                                                       sc.b[i][U0 / 4], U0 % 4, sc.a[j][U0 / 4]);
        }
        if constexpr (F::F16) {
          // fp16: the fragment reads spread over the tile's MFMAs, each copy one MFMA after its
          // share of them (faster than all after the first MFMA, where the compiler puts the MX
          // formats' reads and copies)
          if (k == F::KSTEPS - 1) {
            const int q0 = CP::DPS * i / T::FB, nc = CP::DPS * (i + 1) / T::FB - q0;
            const int f0 = T::F * i / T::FB, nf = T::F * (i + 1) / T::FB - f0;
#pragma unroll
            for (int e = 0; e < nf; e++)
              if ((e * T::FA) / nf == j) next_frag<KIND, T>(c, f0 + e, slot_nxt, na, nb);
#pragma unroll
            for (int e = 0; e < nc; e++)
              if (min(T::FA - 1, (e * T::FA) / nc + 1) == j) stage_copy<KIND>(c, q0 + e, slot_fill, fill_stage);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
    // this tile's share of the stage copies, [DPS*i/FB, DPS*(i+1)/FB), and of the next stage's
    // fragments, list positions [F*i/FB, F*(i+1)/FB) of A0.., B0.. (fp16: placed among the MFMAs)
    if constexpr (!F::F16) {
#pragma unroll
      for (int q = CP::DPS * i / T::FB; q < CP::DPS * (i + 1) / T::FB; q++) stage_copy<KIND>(c, q, slot_fill, fill_stage);
#pragma unroll
      for (int f = T::F * i / T::FB; f < T::F * (i + 1) / T::FB; f++) next_frag<KIND, T>(c, f, slot_nxt, na, nb);
    }
    if constexpr (!F::F16)
      if (S8 == 4 && i == 1) {
        read_raw_scales<KIND, T>(sgrp, raw, 0, c.wm, c.wn, c.r32);
        read_raw_scales<KIND, T>(sgrp, raw1, 1, c.wm, c.wn, c.r32);
      }
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (!F::F16) {
    if (S8 == 2) pack_scales<KIND, T>(raw1, sc, 1, c.h);
    if (S8 == 6) pack_scales<KIND, T>(raw, sc, 0, c.h);
  }
}

template <int KIND, int WAVES_M, int BN_, int F8A, int F8B>
__global__ __launch_bounds__(256, 1) void gemm_ring_kernel(Args p) {
  using F = RingFmt<KIND>;
  using T = RingTile<WAVES_M, BN_>;
  using CP = RingCopies<KIND, T>;
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
  // row bytes (fp16 B: a K-row of N columns)
  const uint32_t RBA = F::F16 ? 2u * (uint32_t)p.K : F::F6 ? (uint32_t)p.K / 4u * 3u : (uint32_t)p.K / (F::A4 ? 2 : 1);
  const uint32_t RBB = F::F16 ? 2u * (uint32_t)p.N : F::F6 ? (uint32_t)p.K / 4u * 3u : (uint32_t)p.K / (F::B4 ? 2 : 1);
  const uint32_t nblk = (uint32_t)p.K / 32;                                                   // K-blocks
  const int nst = p.K / F::ELEMS, ngroups = nst / GROUP;

  // Direct copies. Copy k of this wave in a stage is stage instruction i = wave + 4k, which fills
  // 1 KB of the slot at i * 1024: A rows for i < NI_A, then B rows. With 64-byte rows it covers 16
  // rows, lane l filling physical chunk l%4 of row l/4 (logical chunk (l%4) ^ ((l/16) & 3)); with
  // 32-byte rows 32 rows, lane l filling physical chunk l%2 of row l/2 (logical (l%2) ^ ((l/16) & 1)).
  // Each copy gets its own buffer resource over its rows (clamped to the matrix, empty past the
  // tile), so one lane offset per operand serves all of them and rows past the edge read as zero
  // (their outputs are never stored).
  // fp16 B: B copy b (instruction NI_A + b) fills K-rows 2b and 2b+1 of the stage, 512 bytes each
  // (columns n0..n0+255; N % 256 == 0), lane l filling physical chunk l%32 of row 2b + l/32 from
  // logical chunk (l%32) ^ 4(row & 3); row & 3 = 2(wave & 1) + l/32 for every copy of the wave. Its
  // resource starts at row 2b of the tile's columns and runs to the end of B; the stage offset moves
  // 32 rows down.
  Ctx c;
  c.wave = wave;
  c.wm = wm;
  c.wn = wn;
  c.r32 = r32;
  c.h = h;
  c.nst = nst;
  c.ngroups = ngroups;
  const uint32_t l = (uint32_t)lane;
  const uint32_t off64 = 16u * ((l & 3) ^ ((l >> 4) & 3)), off32 = 16u * ((l & 1) ^ ((l >> 4) & 1));
  c.voff_a = F::SRB_A == 64 ? (l >> 2) * RBA + off64 : (l >> 1) * RBA + off32;
  c.voff_b = F::SRB_B == 64 ? (l >> 2) * RBB + off64 : (l >> 1) * RBB + off32;
  if constexpr (F::F6) {  // lane l fills chunk l%4 of row l/4 with 12-byte piece (l%4) ^ ((l/16) & 3)
    const uint32_t pc = 12u * ((l & 3) ^ ((l >> 4) & 3));
    c.voff_a = (l >> 2) * RBA + pc;
    c.voff_b = (l >> 2) * RBB + pc;
  }
  c.bstage = 32u * RBB;
  if constexpr (F::F16) {
    c.voff_b = (l >> 5) * RBB + 16u * ((l & 31) ^ (8u * ((uint32_t)wave & 1) + 4u * (l >> 5)));
    const uint32_t g16 = l >> 4, i16 = l & 15, y = i16 >> 2;
#pragma unroll
    for (int i = 0; i < T::FB; i++) {
      const uint32_t cc = 4u * (uint32_t)(T::FB * wn + i) + 2u * (g16 & 1) + ((i16 & 3) >> 1);
      c.bt_off[i] = (8u * (g16 >> 1) + y) * 512u + 16u * (cc ^ (4u * y)) + 8u * (i16 & 1);
    }
  }
#pragma unroll
  for (int k = 0; k < CP::DPS; k++) {
    const int i = wave + 4 * k;
    const bool isA = k < F::NI_A / 4;
    const int rpi = F::CPYB / (isA ? F::SRB_A : F::SRB_B);  // rows per instruction (16 or 32)
    const int r0 = rpi * (isA ? i : i - F::NI_A), rows = isA ? rows_a : rows_b;
    const uint32_t rb = isA ? RBA : RBB;
    const int nr = max(0, min(rpi, rows - r0));
    const uint8_t* base = (isA ? p.A + (int64_t)m0 * rb : p.B + (int64_t)n0 * rb) + (int64_t)(nr ? r0 : 0) * rb;
    c.rdata[k] = make_rsrc(base, (uint32_t)nr * rb);
    if constexpr (F::F16) {
      if (!isA) {
        const int64_t start = (int64_t)2 * (i - F::NI_A) * RBB + 2 * (int64_t)n0;
        c.rdata[k] = make_rsrc(p.B + start, (uint32_t)((int64_t)p.K * RBB - start));
      }
    }
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
  if constexpr (!F::F16) issue_scales<KIND>(c, sgrp, 0);
  for (int t = 0; t < 3 && t < nst; t++) {
    char* slot = t == 0 ? slot0 : (t == 1 ? slot1 : slot2);
#pragma unroll
    for (int k = 0; k < CP::DPS; k++) stage_copy<KIND>(c, k, slot, (uint32_t)t);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): prologue copies of this wave
  raw_barrier();
  v8i xa[T::FA], xb[T::FB], ya[T::FA], yb[T::FB];
  Scales<KIND, T> sc;
  RawScales<KIND, T> raw, raw1;
  if constexpr (!F::F16) {
    read_raw_scales<KIND, T>(sgrp, raw, 0, wm, wn, r32);
    pack_scales<KIND, T>(raw, sc, 0, h);
    read_raw_scales<KIND, T>(sgrp, raw1, 1, wm, wn, r32);
    pack_scales<KIND, T>(raw1, sc, 1, h);
  }
#pragma unroll
  for (int j = 0; j < T::FA; j++) {
    if constexpr (F::F6) xa[j] = read_frag6(slot0, row_a<T>(j, wm, r32), h);
    else xa[j] = read_frag<F::SRB_A>(slot0, row_a<T>(j, wm, r32), h);
  }
#pragma unroll
  for (int i = 0; i < T::FB; i++) {
    if constexpr (F::F6) xb[i] = read_frag6(slot0 + BM * F::SRB_A, row_b<T>(i, wn, r32), h);
    else if constexpr (F::F16) xb[i] = read_frag_bt(slot0 + BM * F::SRB_A, c.bt_off[i]);
    else xb[i] = read_frag<F::SRB_B>(slot0 + BM * F::SRB_A, row_b<T>(i, wn, r32), h);
  }

  // Stage t uses slot t%4 (t = 8g + s: slot s%4); even stages compute from x*, odd from y*.
  for (int g = 0; g < ngroups; g++) {
    ring_stage<KIND, T, 0, F8A, F8B>(c, g, sgrp, xa, xb, ya, yb, slot1, slot3, sc, raw, raw1, acc);
    ring_stage<KIND, T, 1, F8A, F8B>(c, g, sgrp, ya, yb, xa, xb, slot2, slot0, sc, raw, raw1, acc);
    ring_stage<KIND, T, 2, F8A, F8B>(c, g, sgrp, xa, xb, ya, yb, slot3, slot1, sc, raw, raw1, acc);
    ring_stage<KIND, T, 3, F8A, F8B>(c, g, sgrp, ya, yb, xa, xb, slot0, slot2, sc, raw, raw1, acc);
    ring_stage<KIND, T, 4, F8A, F8B>(c, g, sgrp, xa, xb, ya, yb, slot1, slot3, sc, raw, raw1, acc);
    ring_stage<KIND, T, 5, F8A, F8B>(c, g, sgrp, ya, yb, xa, xb, slot2, slot0, sc, raw, raw1, acc);
    ring_stage<KIND, T, 6, F8A, F8B>(c, g, sgrp, xa, xb, ya, yb, slot3, slot1, sc, raw, raw1, acc);
    ring_stage<KIND, T, 7, F8A, F8B>(c, g, sgrp, ya, yb, xa, xb, slot0, slot2, sc, raw, raw1, acc);
  }

  // The last stages queued copies of stage nst-1 into free slots: let them land, and let every
  // wave finish with the ring, before the slots are reused for the output.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  raw_barrier();

  // Epilogue. The lane holds C[m0 + 32*FA*wm + 32j + r32][n0 + 32*FB*wn + 32i + 8q + 4h + e] in
  // acc[i][j][4q + e]: 8 bytes per row, so storing straight from registers would write each
  // 128-byte line of C in pieces from several instructions. Instead each wave converts to fp16 into
  // its own slot, 64 rows (two A tiles) at a time with rows padded by 8 bytes (the 8-byte writes of
  // 32 rows then fall on distinct banks), and writes the rows back as 16-byte pieces, consecutive
  // lanes along a row.
  char* stage = wave == 0 ? slot0 : (wave == 1 ? slot1 : (wave == 2 ? slot2 : slot3));
  constexpr int WCOLS = 32 * T::FB;            // columns of the wave's block
  constexpr int EROW = 2 * WCOLS + 8;          // staged row pitch, bytes
  constexpr int LPR = WCOLS / 8;               // 16-byte pieces per row
  constexpr int JP = T::FA < 2 ? T::FA : 2;    // A tiles per pass
  constexpr int PIECES = 32 * JP * LPR;        // per pass: a multiple of 64
  static_assert(PIECES % 64 == 0 && 32 * JP * EROW <= SLOT && T::FA % JP == 0, "epilogue staging");
  const bool rows16 = (p.N & 7) == 0;          // row starts 16-byte aligned
  if (p.relu) {  // (one uniform branch, not a select per element)
#pragma unroll
    for (int i = 0; i < T::FB; i++)
#pragma unroll
      for (int j = 0; j < T::FA; j++)
#pragma unroll
        for (int e = 0; e < 16; e++) acc[i][j][e] = fmaxf(acc[i][j][e], 0.0f);
  }
#pragma unroll
  for (int j0 = 0; j0 < T::FA; j0 += JP) {
#pragma unroll
    for (int jj = 0; jj < JP; jj++)
#pragma unroll
      for (int i = 0; i < T::FB; i++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          v4h o;
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const float v = acc[i][j0 + jj][4 * q + e];
            o[e] = (_Float16)v;
          }
          *reinterpret_cast<v4h*>(stage + (32 * jj + r32) * EROW + (32 * i + 8 * q + 4 * h) * 2) = o;
        }
#pragma unroll
    for (int s0 = 0; s0 < PIECES; s0 += 64) {
      const int piece = s0 + lane, lr = piece / LPR, cp = piece % LPR;
      const char* src = stage + lr * EROW + 16 * cp;
      const v4h lo = *reinterpret_cast<const v4h*>(src), hi = *reinterpret_cast<const v4h*>(src + 8);
      const int m = m0 + 32 * T::FA * wm + 32 * j0 + lr, n = n0 + WCOLS * wn + 8 * cp;
      if (m < p.M) {
        // non-temporal stores: C streams out without displacing the A and B panels that other tiles
        // still read from the L2 and the Infinity Cache
        _Float16* dst = p.C + (int64_t)m * p.N + n;
        if (n + 8 <= p.N) {
          if (rows16) {
            __builtin_nontemporal_store(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7),
                                        reinterpret_cast<v8h*>(dst));
          } else {
            __builtin_nontemporal_store(lo, reinterpret_cast<v4h*>(dst));
            __builtin_nontemporal_store(hi, reinterpret_cast<v4h*>(dst + 4));
          }
        } else if (n + 4 <= p.N) {
          __builtin_nontemporal_store(lo, reinterpret_cast<v4h*>(dst));
        }
      }
    }
  }
}


// ---- 8-wave ping-pong GEMM with 128-byte stage rows ---------------------------------------------
// Measured on gfx950: direct global->LDS copies move about 30 bytes per clock per CU when each row
// contributes a 64-byte run to a copy instruction, and about 58 when it contributes 128 bytes (a
// whole cache line), whatever the number of waves issuing. The ring above stages 64 bytes of every
// row, and its copies, not its MFMAs or fragment reads, set its speed. This kernel stages 128 bytes
// of every row per slot (two slots of 256 + 256 rows, 64 KB each) and hides the shorter look-ahead
// with two waves per SIMD that take turns:
//  - Each SIMD runs waves w and w+4 of the workgroup (measured: the dispatcher places them so).
//    While one issues the MFMAs of a step from registers (its C phase), the other queues copies
//    and reads its fragments of the next step (its L phase); waves 4..7 run one phase behind waves
//    0..3, and a barrier separates consecutive phases, so each barrier pairs a C phase of one group
//    with an L phase of the other and each SIMD's matrix core always has a wave with MFMAs to issue.
//  - Tile 256 x 256; wave w owns rows 128(w%2).. and columns 64(w/2).., 4 x 2 MFMA tiles of
//    32 x 32: 128 accumulator registers, so two waves fit a SIMD's register file.
//  - A step is 64 bytes of every row (one 32x32x64 K-step of E4M3, two of E2M1); slot m holds steps
//    2m and 2m+1. Rows in a slot are 128 bytes, 16-byte chunk c of row r stored at c ^ ((r >> 1) & 7)
//    (the 16 rows of a quarter-wave fragment read then cover all 64 banks once). A copy instruction
//    fills 1 KB: 8 rows x 128 bytes, lane l filling physical chunk l%8 of row l/8; wave w issues
//    instructions w + 8k (k < 4: A rows, k >= 4: B rows) of a slot.
//  - fp16 (KIND 4): a step is 32 K (64 bytes of an A row, two 32x32x16 fp16 K-steps) with no scale
//    plane; B is K x N, staged per slot as 64 K-rows of the tile's 256 columns and read into MFMA
//    fragments by transposing LDS reads (pp_read_ab16).
//  - Two steps of a wave (pp_step2): the B rows of a slot are read in the first L phase, so they can
//    be refilled one step earlier and get three steps to land (the A rows two); reads and copies are
//    split evenly between the two L phases.
//  - Scales: groups of 16 bytes per row (8 K-steps: 8 E4M3 steps or 4 E2M1 steps), double buffered;
//    group q+2 is copied (one 1 KB copy per wave) in the group's second step into the buffer of
//    group q, whose scales were packed into registers in the step before group q began; group q+1
//    is read and packed in group q's last step.
//  - Both groups pass the same number of barriers: 1 after the prologue, 2 per step, and one extra
//    (at the start for waves 4-7, at the end for waves 0-3), then the epilogue's.
template <int KIND>
struct PPFmt {
  enum : int {
    G = 8 / RingFmt<KIND>::KSTEPS,  // steps per scale group
    SLOT2 = 512 * 128,              // bytes of one slot: 256 A + 256 B rows of 128 bytes
    SBUF = 512 * 16                 // bytes of one scale buffer
  };
  static_assert(KIND >= 0 && KIND <= 5,
                "ping-pong GEMM: byte pairs, E2M1 x E2M1, byte x E2M1 mixes, fp16 x fp16, FP6 pairs");
};

struct PPCtx {
  rsrc_t rdata[8];
  rsrc_t rscale;
  uint32_t voff, svoff;
  // LDS byte offsets within a slot of the lane's chunk h of its first A and B fragment rows (A: row
  // 128 wm + r32; B: row 64 wn + r32 of the B region; swizzled). Chunk h + k (k = 0, 2, 4, 6) of the
  // same row is at that offset XOR 16k: the swizzle only permutes the chunks of a row. Also the
  // offsets of its scale rows within a scale buffer.
  uint32_t fa0, fb0, sc_a, sc_b;
  // FP6: the lane's 8-byte pieces t = 0..2 of step hs of a row (bytes 48 hs + 24 h + 8 t of the row's
  // 96 data bytes), as offsets from the row's first byte (fa0 / fb0 are then row starts)
  uint32_t f6o[2][3];
  // fp16 (KIND 4): B is K x N, N-contiguous, staged per slot as 64 K-rows of 512 bytes (the tile's
  // 256 columns; 16-byte chunk c of K-row k at chunk c ^ 4 (k & 3)): the lane offset of its B-row
  // copies, the bytes between the B rows of consecutive slots, and the lane's transposing-read
  // offsets of its two B tiles in a step's 32 K-rows
  uint32_t voff_b, bslot, bt_off[2];
  int wave, wm, wn, r32, h, nst, ngroups, nslots;
  // A given as fp16 and quantised on load: resource over the tile's fp16 A rows; this thread's row
  // rq = tid / 2 and block bq = tid % 2 of each step (64 K-elements = 2 blocks of 32) it quantises:
  // its source offset, its slot row offset and chunk swizzle; the lane's A-scale read offsets
  rsrc_t ra16;
  uint32_t qa_voff, qa_row, qa_sw, qa_asc_w, qa_asc_r;
  int qa_bq;
};

MX_DEV uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_ptr_t)p; }

// 16-byte LDS reads as inline assembly: the compiler then neither waits for the direct copies in
// flight (it cannot tell which slot they fill) nor keeps one address register per slot and
// fragment; the waits are explicit (lgkmcnt(0) at the end of each L phase). Early-clobber outputs:
// a destination must not share a register with a later read's address. Tiles j and j+1 are 32
// rows = 4096 bytes apart.
template <int OFF>
MX_DEV void pp_read4(v4i& d0, v4i& d1, v4i& d2, v4i& d3, uint32_t a0, uint32_t a1) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:%6\n"
      "ds_read_b128 %1, %5 offset:%6\n"
      "ds_read_b128 %2, %4 offset:%7\n"
      "ds_read_b128 %3, %5 offset:%7"
      : "=&v"(d0), "=&v"(d1), "=&v"(d2), "=&v"(d3)
      : "v"(a0), "v"(a1), "i"(OFF), "i"(OFF + 4096));
}
MX_DEV void pp_read1(v4i& d, uint32_t a) { asm volatile("ds_read_b128 %0, %1" : "=&v"(d) : "v"(a)); }
// FP6: the same four reads of 12 bytes (a piece of a row's step is 12 bytes in its 16-byte chunk).
typedef int v3i __attribute__((ext_vector_type(3)));
template <int OFF>
MX_DEV void pp_read4_96(v3i& d0, v3i& d1, v3i& d2, v3i& d3, uint32_t a0, uint32_t a1) {
  asm volatile(
      "ds_read_b96 %0, %4 offset:%6\n"
      "ds_read_b96 %1, %5 offset:%6\n"
      "ds_read_b96 %2, %4 offset:%7\n"
      "ds_read_b96 %3, %5 offset:%7"
      : "=&v"(d0), "=&v"(d1), "=&v"(d2), "=&v"(d3)
      : "v"(a0), "v"(a1), "i"(OFF), "i"(OFF + 4096));
}
MX_DEV v8i cat6(v3i lo, v3i hi) {
  const v4i a = __builtin_shufflevector(lo, lo, 0, 1, 2, -1), b = __builtin_shufflevector(hi, hi, 0, 1, 2, -1);
  return __builtin_shufflevector(a, b, 0, 1, 2, 4, 5, 6, -1, -1);
}
MX_DEV v8i cat8(v4i lo, v4i hi) { return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7); }

// The copies of slot m (its steps 2m, 2m+1: bytes 128m.. of every row; FP6: the 96 bytes 96m.. in
// logical chunks 0..5 of the 128-byte LDS row, chunks 6 and 7 unused) into `dst`: the 4 of its A
// rows (HALF 0) or of its B rows (HALF 1). Byte A x E2M1 B (KIND 2): a step is 32 bytes of a B row,
// so B rows are copied 128 bytes (steps 4m..4m+3) at a time, m then counting those 4-step pairs; the
// same for the A rows of E2M1 A x byte B (KIND 3).
// The loads bypass the CU's L1 (sc0): no byte is read twice by one CU (measured about 3% faster at
// the MXFP8 prefill shape).
template <int KIND, int HALF>
MX_DEV void pp_slot_copies(const PPCtx& c, char* dst, uint32_t m) {
#pragma unroll
  for (int k = 4 * HALF; k < 4 * HALF + 4; k++) {
    if constexpr (KIND == 5)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rdata[k], (lds_ptr_t)(dst + (c.wave + 8 * k) * 1024), 16, c.voff,
                                               96u * m, 0, 1);
    else if constexpr (KIND == 4 && HALF == 1)  // (the slot's K rows in the lane offset: see the set-up)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rdata[k], (lds_ptr_t)(dst + (c.wave + 8 * k) * 1024), 16,
                                               c.voff_b + m * c.bslot, 0, 0, 1);
    else if constexpr ((KIND == 2 || KIND == 3) && HALF == 1)  // B rows of a mix (KIND 2: E2M1, m counts pairs)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rdata[k], (lds_ptr_t)(dst + (c.wave + 8 * k) * 1024), 16, c.voff_b,
                                               128u * m, 0, 1);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rdata[k], (lds_ptr_t)(dst + (c.wave + 8 * k) * 1024), 16, c.voff,
                                               128u * m, 0, 1);
  }
}

MX_DEV void pp_scale_copy(const PPCtx& c, char* sbuf, int q) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rscale, (lds_ptr_t)(sbuf + c.wave * 1024), 16, c.svoff, 16 * q, 0, 0);
}

// The lane's packed scales of a group from the 16 bytes r of its row: byte u%4 of dword u/4 is its
// scale (K-block h) for K-step u of the group.
MX_DEV void pp_pack(const v4i r, int h, uint32_t (&out)[2]) {
  const uint32_t sel = h ? 0x07050301u : 0x06040200u;
  out[0] = __builtin_amdgcn_perm((uint32_t)r[1], (uint32_t)r[0], sel);
  out[1] = __builtin_amdgcn_perm((uint32_t)r[3], (uint32_t)r[2], sel);
}

// MFMAs of one step from the fragments f (A tiles 0..3, B tiles 4, 5) with the group's packed
// scales; U0 = first K-step of the step within its scale group.
// With the A operand quantised on load (QA) the A scale of each tile is one byte per step, in the
// low byte of sq[j] (op_sel 0). FC: the MFMA format codes of the operands, A's in bits 0-3 and B's in
// bits 4-7 (KIND 0: 0 = E4M3, 1 = E5M2, which share the byte layout; KIND 5: 2 = E2M3, 3 = E3M2).
template <int KIND, int U0, bool QA = false, int FC = 0>
MX_DEV void pp_mfmas(const v8i (&f)[6], const uint32_t (&sa)[4][2], const uint32_t (&sb)[2][2], v16f (&acc)[2][4],
                     const uint32_t* sq = nullptr) {
  using F = RingFmt<KIND>;
#pragma unroll
  for (int k = 0; k < F::KSTEPS; k++)
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if constexpr (F::F16) {
          const v8h bk = __builtin_bit_cast(v8h, k ? __builtin_shufflevector(f[4 + i], f[4 + i], 4, 5, 6, 7)
                                                   : __builtin_shufflevector(f[4 + i], f[4 + i], 0, 1, 2, 3));
          const v8h ak = __builtin_bit_cast(v8h, k ? __builtin_shufflevector(f[j], f[j], 4, 5, 6, 7)
                                                   : __builtin_shufflevector(f[j], f[j], 0, 1, 2, 3));
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bk, ak, acc[i][j], 0, 0, 0);
        } else if constexpr (F::FP4) {
          const v8i bk = k ? __builtin_shufflevector(f[4 + i], f[4 + i], 4, 5, 6, 7, -1, -1, -1, -1)
                           : __builtin_shufflevector(f[4 + i], f[4 + i], 0, 1, 2, 3, -1, -1, -1, -1);
          const v8i ak = k ? __builtin_shufflevector(f[j], f[j], 4, 5, 6, 7, -1, -1, -1, -1)
                           : __builtin_shufflevector(f[j], f[j], 0, 1, 2, 3, -1, -1, -1, -1);
          if (k == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bk, ak, acc[i][j], 4, 4, U0 % 4, sb[i][U0 / 4],
                                                                         U0 % 4, sa[j][U0 / 4]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bk, ak, acc[i][j], 4, 4, (U0 + 1) % 4, sb[i][(U0 + 1) / 4], (U0 + 1) % 4, sa[j][(U0 + 1) / 4]);
        } else if constexpr (QA) {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f[4 + i], f[j], acc[i][j], 0, 0, U0 % 4,
                                                                       sb[i][U0 / 4], 0, sq[j]);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f[4 + i], f[j], acc[i][j], FC >> 4, FC & 15,
                                                                       U0 % 4, sb[i][U0 / 4], U0 % 4, sa[j][U0 / 4]);
        }
      }
}

MX_DEV void pp_phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  raw_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Fragment reads of a slot. Step hs (0, 1) of the slot is chunks 4 hs + h (lo) and 4 hs + 2 + h (hi)
// of each row. pp_read_ab: A tiles 0..3 and B tiles 0, 1 of step HS into f, plus B tiles 0, 1 of
// step 1 into yb when YB; pp_read_a: A tiles 0..3 of step 1 into f. Each ends with lgkmcnt(0).
MX_DEV uint32_t pp_base(const char* slot) {
  // (an opaque copy of the slot address: otherwise the compiler keeps the sums base + offset of both
  // slots in registers across the loop, which do not fit beside the accumulators and fragments)
  uint32_t base = lds_addr(slot);
  asm volatile("" : "+s"(base));
  return base;
}
// FP6 (KIND 5): the lane's fragment of step hs is bytes 48 hs + 24 h .. + 23 of its row's 96 data
// bytes: three 8-byte reads at the lane's offsets f6o[hs][0..2] (they straddle the swizzled 16-byte
// chunks), tiles 4096 bytes apart. The reads land in dwords 0-5 of the MFMA operand.
typedef int v2i __attribute__((ext_vector_type(2)));
template <int OFF>
MX_DEV void pp_read3_64(v2i& d0, v2i& d1, v2i& d2, uint32_t a0, uint32_t a1, uint32_t a2) {
  asm volatile(
      "ds_read_b64 %0, %3 offset:%6\n"
      "ds_read_b64 %1, %4 offset:%6\n"
      "ds_read_b64 %2, %5 offset:%6"
      : "=&v"(d0), "=&v"(d1), "=&v"(d2)
      : "v"(a0), "v"(a1), "v"(a2), "i"(OFF));
}
MX_DEV v8i cat3x2(v2i x, v2i y, v2i z) {
  const v4i xy = __builtin_shufflevector(x, y, 0, 1, 2, 3), zz = __builtin_shufflevector(z, z, 0, 1, -1, -1);
  return __builtin_shufflevector(xy, zz, 0, 1, 2, 3, 4, 5, -1, -1);
}
template <int HS, int NT>
MX_DEV void pp_frags6(const PPCtx& c, uint32_t row, v8i* f) {
  const uint32_t a0 = row + c.f6o[HS][0], a1 = row + c.f6o[HS][1], a2 = row + c.f6o[HS][2];
  v2i r[NT][3];
  pp_read3_64<0>(r[0][0], r[0][1], r[0][2], a0, a1, a2);
  pp_read3_64<4096>(r[1][0], r[1][1], r[1][2], a0, a1, a2);
  if constexpr (NT == 4) {
    pp_read3_64<8192>(r[2][0], r[2][1], r[2][2], a0, a1, a2);
    pp_read3_64<12288>(r[3][0], r[3][1], r[3][2], a0, a1, a2);
  }
#pragma unroll
  for (int t = 0; t < NT; t++) f[t] = cat3x2(r[t][0], r[t][1], r[t][2]);
}
template <int HS, bool YB>
MX_DEV void pp_read_ab6(const PPCtx& c, const char* slot, v8i (&f)[6], v8i (&yb)[2]) {
  const uint32_t base = pp_base(slot);
  pp_frags6<HS, 4>(c, base + c.fa0, &f[0]);
  pp_frags6<HS, 2>(c, base + c.fb0, &f[4]);
  if (YB) pp_frags6<1, 2>(c, base + c.fb0, &yb[0]);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
}
MX_DEV void pp_read_a6(const PPCtx& c, const char* slot, v8i (&f)[6]) {
  pp_frags6<1, 4>(c, pp_base(slot) + c.fa0, &f[0]);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
}
template <int HS, bool YB>
MX_DEV void pp_read_ab(const PPCtx& c, const char* slot, v8i (&f)[6], v8i (&yb)[2]) {
  const uint32_t base = pp_base(slot), a = base + c.fa0, b = base + c.fb0;
  v4i r[16];
  pp_read4<0>(r[0], r[1], r[2], r[3], a ^ (64u * HS), a ^ (64u * HS + 32u));
  pp_read4<8192>(r[4], r[5], r[6], r[7], a ^ (64u * HS), a ^ (64u * HS + 32u));
  pp_read4<0>(r[8], r[9], r[10], r[11], b ^ (64u * HS), b ^ (64u * HS + 32u));
  if (YB) pp_read4<0>(r[12], r[13], r[14], r[15], b ^ 64u, b ^ 96u);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < 6; t++) f[t] = cat8(r[2 * t], r[2 * t + 1]);
  if (YB) {
    yb[0] = cat8(r[12], r[13]);
    yb[1] = cat8(r[14], r[15]);
  }
}
// Byte A x E2M1 B (KIND 2): A fragments of step 0 of the slot as pp_read_ab's; B rows hold 4 steps
// of 32 bytes (128 bytes: a 4-step pair), and the E2M1 operand of step s is the lane's 16 bytes (its
// K-block h: 32 nibbles) in chunk 2s + h. B tiles 0, 1 of steps S0 and S0 + 1 of the pair into f[4],
// f[5] and yb; the upper four dwords of an E2M1 operand are not read by the MFMA.
template <int S0>
MX_DEV void pp_read_ab_m4(const PPCtx& c, const char* slot, const char* bbuf, v8i (&f)[6], v8i (&yb)[2]) {
  const uint32_t a = pp_base(slot) + c.fa0, b = pp_base(bbuf) + c.fb0;
  v4i r[8], t[4];
  pp_read4<0>(r[0], r[1], r[2], r[3], a, a ^ 32u);
  pp_read4<8192>(r[4], r[5], r[6], r[7], a, a ^ 32u);
  pp_read4<0>(t[0], t[1], t[2], t[3], b ^ (32u * S0), b ^ (32u * (S0 + 1)));
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 4; j++) f[j] = cat8(r[2 * j], r[2 * j + 1]);
  f[4] = __builtin_shufflevector(t[0], t[0], 0, 1, 2, 3, -1, -1, -1, -1);
  f[5] = __builtin_shufflevector(t[2], t[2], 0, 1, 2, 3, -1, -1, -1, -1);
  yb[0] = __builtin_shufflevector(t[1], t[1], 0, 1, 2, 3, -1, -1, -1, -1);
  yb[1] = __builtin_shufflevector(t[3], t[3], 0, 1, 2, 3, -1, -1, -1, -1);
}
// E2M1 A x byte B (KIND 3): A rows hold 4 steps of 32 bytes; A tiles 0..3 of step S of the pair are
// chunk 2S + h of their rows (tiles 0, 2 at a, a + 8192; tiles 1, 3 4096 bytes on).
MX_DEV v8i widen4(v4i t) { return __builtin_shufflevector(t, t, 0, 1, 2, 3, -1, -1, -1, -1); }
template <int S>
MX_DEV void pp_frags_a4(const PPCtx& c, const char* abuf, v4i (&t)[4]) {
  const uint32_t a = (pp_base(abuf) + c.fa0) ^ (32u * S);
  pp_read4<0>(t[0], t[1], t[2], t[3], a, a + 8192u);
}
template <int S0>
MX_DEV void pp_read_ab_a4(const PPCtx& c, const char* abuf, const char* slot, v8i (&f)[6], v8i (&yb)[2]) {
  const uint32_t b = pp_base(slot) + c.fb0;
  v4i t[4], r[8];
  pp_frags_a4<S0>(c, abuf, t);
  pp_read4<0>(r[0], r[1], r[2], r[3], b, b ^ 32u);
  pp_read4<0>(r[4], r[5], r[6], r[7], b ^ 64u, b ^ 96u);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
  f[0] = widen4(t[0]);
  f[1] = widen4(t[2]);
  f[2] = widen4(t[1]);
  f[3] = widen4(t[3]);
  f[4] = cat8(r[0], r[1]);
  f[5] = cat8(r[2], r[3]);
  yb[0] = cat8(r[4], r[5]);
  yb[1] = cat8(r[6], r[7]);
}
template <int S>
MX_DEV void pp_read_a_a4(const PPCtx& c, const char* abuf, v8i (&f)[6]) {
  v4i t[4];
  pp_frags_a4<S>(c, abuf, t);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
  f[0] = widen4(t[0]);
  f[1] = widen4(t[2]);
  f[2] = widen4(t[1]);
  f[3] = widen4(t[3]);
}
// fp16: A fragments are E4M3's (chunks h and h + 2 of the step: K-steps 0 and 1 of the 32x32x16
// fp16 MFMA); a B fragment is four transposing 8-byte reads of its tile (K-rows 8h + y, + 4, + 16,
// + 20 of the step: two K-steps of 8 rows each), the second step's rows 16384 bytes on.
template <int OFF>
MX_DEV void pp_read_tr4(v2i& d0, v2i& d1, v2i& d2, v2i& d3, uint32_t a) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4 offset:%5\n"
      "ds_read_b64_tr_b16 %1, %4 offset:%6\n"
      "ds_read_b64_tr_b16 %2, %4 offset:%7\n"
      "ds_read_b64_tr_b16 %3, %4 offset:%8"
      : "=&v"(d0), "=&v"(d1), "=&v"(d2), "=&v"(d3)
      : "v"(a), "i"(OFF), "i"(OFF + 2048), "i"(OFF + 8192), "i"(OFF + 10240));
}
MX_DEV v8i cat4x2(v2i a, v2i b, v2i c, v2i d) {
  const v4i ab = __builtin_shufflevector(a, b, 0, 1, 2, 3), cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return cat8(ab, cd);
}
template <int HS, bool YB>
MX_DEV void pp_read_ab16(const PPCtx& c, const char* slot, v8i (&f)[6], v8i (&yb)[2]) {
  const uint32_t base = pp_base(slot), a = base + c.fa0, b = base + (uint32_t)BM * 128u;
  const uint32_t b0 = b + c.bt_off[0], b1 = b + c.bt_off[1];
  v4i r[8];
  v2i t[4][4];
  pp_read4<0>(r[0], r[1], r[2], r[3], a ^ (64u * HS), a ^ (64u * HS + 32u));
  pp_read4<8192>(r[4], r[5], r[6], r[7], a ^ (64u * HS), a ^ (64u * HS + 32u));
  pp_read_tr4<16384 * HS>(t[0][0], t[0][1], t[0][2], t[0][3], b0);
  pp_read_tr4<16384 * HS>(t[1][0], t[1][1], t[1][2], t[1][3], b1);
  if (YB) {
    pp_read_tr4<16384>(t[2][0], t[2][1], t[2][2], t[2][3], b0);
    pp_read_tr4<16384>(t[3][0], t[3][1], t[3][2], t[3][3], b1);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 4; j++) f[j] = cat8(r[2 * j], r[2 * j + 1]);
  f[4] = cat4x2(t[0][0], t[0][1], t[0][2], t[0][3]);
  f[5] = cat4x2(t[1][0], t[1][1], t[1][2], t[1][3]);
  if (YB) {
    yb[0] = cat4x2(t[2][0], t[2][1], t[2][2], t[2][3]);
    yb[1] = cat4x2(t[3][0], t[3][1], t[3][2], t[3][3]);
  }
}
MX_DEV void pp_read_a(const PPCtx& c, const char* slot, v8i (&f)[6]) {
  const uint32_t a = pp_base(slot) + c.fa0;
  v4i r[8];
  pp_read4<0>(r[0], r[1], r[2], r[3], a ^ 64u, a ^ 96u);
  pp_read4<8192>(r[4], r[5], r[6], r[7], a ^ 64u, a ^ 96u);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < 4; t++) f[t] = cat8(r[2 * t], r[2 * t + 1]);
}

// Raw scale rows of a group from a scale buffer, packed: sa (A tiles 0..3), sb (B tiles 0, 1).
MX_DEV void pp_read_scales(const PPCtx& c, const char* sbuf, uint32_t (&sa)[4][2], uint32_t (&sb)[2][2]) {
  uint32_t sbase = lds_addr(sbuf);
  asm volatile("" : "+s"(sbase));
  v4i rs[6];
#pragma unroll
  for (int j = 0; j < 4; j++) pp_read1(rs[j], sbase + c.sc_a + 512u * j);
#pragma unroll
  for (int i = 0; i < 2; i++) pp_read1(rs[4 + i], sbase + c.sc_b + 512u * i);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 4; j++) pp_pack(rs[j], c.h, sa[j]);
#pragma unroll
  for (int i = 0; i < 2; i++) pp_pack(rs[4 + i], c.h, sb[i]);
}

// ---- A quantised on load (E4M3 from fp16) ----
// A block of 32 fp16 values becomes 32 E4M3 codes and one E8M0 scale by the rule of mx_pack_run:
// E = clamp(floor(log2 amax) - 8 + 127, 0, 254) from the exact binary exponent of amax (E = 0 for
// amax = 0; 0xFF with zero codes for a block holding Inf or NaN), codes = x * 2^(127-E) rounded to
// the nearest E4M3 value, ties to even, saturating to +-448, sign kept. gfx950's scaled conversion
// v_cvt_scalef32_pk_fp8_f16 (two values per instruction, divided by the scale) gives exactly these
// codes for every fp16 input and every scale such an fp16 block produces (measured against the
// library codec on all 65536 fp16 values and scales 2^-40..2^40), except that it writes NaN
// (S.1111.111) where the scaled value exceeds 464 instead of saturating: those bytes are turned into
// S.1111.110 (+-448) below. Inputs are upcast exactly, so the codes equal mx_pack_run's on the fp32
// copy of the fp16 activations.
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
typedef short v2s16 __attribute__((ext_vector_type(2)));
typedef _Float16 v2f16 __attribute__((ext_vector_type(2)));

MX_DEV void qa_block(const v4i (&w)[4], v4i& lo, v4i& hi, uint32_t& ebyte) {
  v2u16 m = {0, 0};
#pragma unroll
  for (int d = 0; d < 16; d++) {
    const uint32_t e = (uint32_t)w[d / 4][d % 4] & 0x7FFF7FFFu;
    m = __builtin_elementwise_max(m, __builtin_bit_cast(v2u16, e));
  }
  const uint32_t m0 = m[0], m1 = m[1];
  const uint32_t a = m0 > m1 ? m0 : m1;  // amax as fp16 magnitude bits
  const bool nonfinite = a >= 0x7C00u;
  // floor(log2 amax): the exponent of its exact fp32 copy (fp16 subnormals are normal in fp32);
  // branch-free, so the loop body stays one basic block
  const float af = (float)__builtin_bit_cast(_Float16, (unsigned short)a);
  const int fl = (int)((__builtin_bit_cast(uint32_t, af) >> 23) & 0xFFu) - 127;
  int E = fl - 8 + 127;
  E = E < 0 ? 0 : (E > 254 ? 254 : E);
  E = a == 0u ? 0 : E;
  // (any scale gives +-0 for an all-zero block; 2^(E-127) is a normal fp32 for every fp16 block)
  const float scale = a == 0u ? 1.0f : __builtin_bit_cast(float, (uint32_t)E << 23);
  uint32_t c[8];
#pragma unroll
  for (int k = 0; k < 8; k++) {
    // (elements copied to scalars first: a bit cast applied to an ext-vector element reads element 0)
    const uint32_t e0 = (uint32_t)w[k / 2][2 * (k % 2)], e1 = (uint32_t)w[k / 2][2 * (k % 2) + 1];
    const v2f16 p0 = __builtin_bit_cast(v2f16, e0), p1 = __builtin_bit_cast(v2f16, e1);
    v2s16 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16((v2s16){0, 0}, p0, scale, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(r, p1, scale, true);
    uint32_t x = __builtin_bit_cast(uint32_t, r);
    const uint32_t t = x & 0x7F7F7F7Fu, nan = (t + 0x01010101u) & 0x80808080u;  // bytes S.1111.111
    x ^= nan >> 7;                                                                // -> S.1111.110
    c[k] = nonfinite ? 0u : x;
  }
  lo = (v4i){(int)c[0], (int)c[1], (int)c[2], (int)c[3]};
  hi = (v4i){(int)c[4], (int)c[5], (int)c[6], (int)c[7]};
  ebyte = nonfinite ? 0xFFu : (uint32_t)E;
}

// This thread's fp16 source block of step s (64 bytes at byte 128 s of its row): 4 loads.
MX_DEV void qa_load(const PPCtx& c, int s, v4i (&w)[4]) {
#pragma unroll
  for (int k = 0; k < 4; k++)
    w[k] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(c.ra16, c.qa_voff + 16u * k, 128u * s, 0));
}

// Quantise the block loaded for step s and write its 32 codes into `slot` (half s % 2 of the row:
// chunks 4(s%2) + 2 bq and the next, swizzled) and its scale byte into the step's A-scale entry.
// Inline-assembly stores: the compiler would otherwise wait for every direct copy in flight into
// the slot arrays before them; the L phase's lgkmcnt(0) completes them before its barrier.
MX_DEV void qa_store(const PPCtx& c, int s, const v4i (&w)[4], char* slot, char* asc) {
  v4i lo, hi;
  uint32_t e;
  qa_block(w, lo, hi, e);
  uint32_t base = lds_addr(slot), abase = lds_addr(asc);
  asm volatile("" : "+s"(base), "+s"(abase));
  const uint32_t c0 = 4u * (uint32_t)(s & 1) + 2u * (uint32_t)c.qa_bq;
  const uint32_t a0 = base + c.qa_row + 16u * (c0 ^ c.qa_sw), a1 = base + c.qa_row + 16u * ((c0 + 1u) ^ c.qa_sw);
  const uint32_t ae = abase + 512u * (uint32_t)(s & 3) + c.qa_asc_w;
  asm volatile(
      "ds_write_b128 %0, %3\n"
      "ds_write_b128 %1, %4\n"
      "ds_write_b8 %2, %5"
      :
      : "v"(a0), "v"(a1), "v"(ae), "v"(lo), "v"(hi), "v"(e)
      : "memory");
}

// The lane's A scales of step s (tiles 0..3: rows 128 wm + 32 j + r32, block h), one byte each.
MX_DEV void qa_read_scales(const PPCtx& c, int s, const char* asc, uint32_t (&sq)[4]) {
  uint32_t abase = lds_addr(asc);
  asm volatile("" : "+s"(abase));
  const uint32_t a = abase + 512u * (uint32_t)(s & 3) + c.qa_asc_r;
  asm volatile(
      "ds_read_u8 %0, %4\n"
      "ds_read_u8 %1, %4 offset:64\n"
      "ds_read_u8 %2, %4 offset:128\n"
      "ds_read_u8 %3, %4 offset:192"
      : "=&v"(sq[0]), "=&v"(sq[1]), "=&v"(sq[2]), "=&v"(sq[3])
      : "v"(a));
}

MX_DEV void pp_read_scales_b(const PPCtx& c, const char* sbuf, uint32_t (&sb)[2][2]) {
  uint32_t sbase = lds_addr(sbuf);
  asm volatile("" : "+s"(sbase));
  v4i rs[2];
#pragma unroll
  for (int i = 0; i < 2; i++) pp_read1(rs[i], sbase + c.sc_b + 512u * i);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 2; i++) pp_pack(rs[i], c.h, sb[i]);
}

// Steps u = G*q + S8 and u+1 (S8 even) of a wave of group GR: L_u, C_u, L_{u+1}, C_{u+1}, each
// phase followed by a barrier. Slot u/2 (`slot_cur`) holds both steps; `slot_oth` is the other slot.
//  - L_u reads the wave's fragments of step u and its B fragments of step u+1 (so the B rows of the
//    slot are free after it), and queues the A-row copies of slot u/2 + 1 into the other slot, whose
//    A rows both groups finished reading in L_{u-1}.
//  - L_{u+1} reads the A fragments of step u+1 and queues the B-row copies of slot u/2 + 2 into this
//    slot; at the group's second step it also queues the scale copy of group q+2 into this group's
//    scale buffer (packed in the step before group q began), and at the group's last step it reads
//    and packs the scales of group q+1.
//  - (Past the last slot the copies repeat the last slot, into free rows.)
//  - Slot u/2 + 1 is first read in L_{u+2}: its copies (B rows queued in L_{u-1}, A rows in L_u) must
//    have landed before the barrier ahead of that phase, which ends C_{u+1} for waves 0-3 and L_{u+1}
//    for waves 4-7. Each wave then has queued after them the 4 B-row copies of L_{u+1}, and the scale
//    copy when L_{u+1} is the group's second step: vmcnt(4) or vmcnt(5).
//  - Reads are split 16 + 8 and copies 4 + 4 between the two L phases, and the B rows get three steps
//    to land, the A rows two.
//  - With A quantised on load (QA): instead of A-row copies, every L phase v quantises this thread's
//    block of step v+2 (loaded in the wave's previous L phase) into the slot of step v+2, whose A
//    rows are free since L_{v-1}, and its scale byte into the step's A-scale entry, then loads its
//    block of step v+3. Issue order per L phase: the 4 A loads, then (odd phases) the B-row copies
//    and the scale copy; the wait at the end of the odd step then allows the 12 later A loads and
//    B copies plus the scale copies queued after the slot's B copies.
template <int KIND, int GR, int S8, bool QA, int FC>
MX_DEV void pp_step2(const PPCtx& c, int q, char* slot_cur, char* slot_oth, char* sb_cur, char* sb_nxt,
                     uint32_t (&sa)[4][2], uint32_t (&sb)[2][2], uint32_t (&na)[4][2], uint32_t (&nb)[2][2],
                     v16f (&acc)[2][4], char* asc, v4i (&ld)[4], char* bb, char* bbo) {
  using F = RingFmt<KIND>;
  constexpr int G = PPFmt<KIND>::G;
  constexpr bool SC = KIND != 4;  // a scale plane (fp16 has none)
  // KIND 2: the B rows of steps u..u+3 (u % 4 == 0) sit in the B half of slot (u / 4) % 2 (`bb`); they
  // are read in L_u and L_{u+2}, and the pair two ahead is copied over them in L_{u+3}, so only steps
  // with S8 % 4 == 2 queue B copies.
  // KIND 3: the A rows of steps u..u+3 sit in the A half of slot (u / 4) % 2 (`bb`), read in L_u ..
  // L_{u+3}; the next pair is copied into the other A half (`bbo`, free since L_{u-1}) in L_u when
  // S8 % 4 == 0. The end of a step pair then waits only for copies queued before it (the next
  // pair's A rows have four steps to land).
  constexpr bool M4 = KIND == 2, A4M = KIND == 3;
  constexpr int BCP = M4 ? (S8 % 4 == 2 ? 4 : 0) : 4;  // B copies this wave queues in L_{u+1}
  constexpr int ACP = A4M ? (S8 % 4 == 0 ? 4 : 0) : 0;  // A copies that need not land in this step pair
  constexpr int WAIT = QA ? 12 + (S8 == 2 ? 1 : 0) + (S8 == 0 ? 1 : 0)
                          : ACP + BCP + (SC && (S8 + 1) % G == 1 ? 1 : 0);
  const int u = G * q + S8;
  v8i x[6], y[6];
  uint32_t sq[4];
  // ---- L_u
  if constexpr (QA) {
    qa_store(c, u + 2, ld, slot_oth, asc);       // step u+2: half 0 of the other slot
    qa_load(c, min(u + 3, c.nst - 1), ld);
    qa_read_scales(c, u, asc, sq);
  }
  if constexpr (KIND == 5) pp_read_ab6<0, true>(c, slot_cur, x, *reinterpret_cast<v8i(*)[2]>(&y[4]));
  else if constexpr (KIND == 4) pp_read_ab16<0, true>(c, slot_cur, x, *reinterpret_cast<v8i(*)[2]>(&y[4]));
  else if constexpr (M4) pp_read_ab_m4<S8 % 4>(c, slot_cur, bb, x, *reinterpret_cast<v8i(*)[2]>(&y[4]));
  else if constexpr (A4M) pp_read_ab_a4<S8 % 4>(c, bb, slot_cur, x, *reinterpret_cast<v8i(*)[2]>(&y[4]));
  else pp_read_ab<0, true>(c, slot_cur, x, *reinterpret_cast<v8i(*)[2]>(&y[4]));
  if constexpr (A4M) {
    if constexpr (S8 % 4 == 0) pp_slot_copies<KIND, 0>(c, bbo, (uint32_t)min(u / 4 + 1, c.nslots / 2 - 1));
  } else if constexpr (!QA) {
    pp_slot_copies<KIND, 0>(c, slot_oth, (uint32_t)min(u / 2 + 1, c.nslots - 1));
  }
  pp_phase_barrier();
  // ---- C_u
  pp_mfmas<KIND, F::KSTEPS * S8, QA, FC>(x, sa, sb, acc, sq);
  pp_phase_barrier();
  // ---- L_{u+1}
  if constexpr (QA) {
    qa_store(c, u + 3, ld, slot_oth, asc);       // step u+3: half 1 of the other slot
    qa_load(c, min(u + 4, c.nst - 1), ld);
    qa_read_scales(c, u + 1, asc, sq);
  }
  if constexpr (KIND == 5) pp_read_a6(c, slot_cur, *reinterpret_cast<v8i(*)[6]>(&y[0]));
  else if constexpr (A4M) pp_read_a_a4<S8 % 4 + 1>(c, bb, *reinterpret_cast<v8i(*)[6]>(&y[0]));
  else pp_read_a(c, slot_cur, *reinterpret_cast<v8i(*)[6]>(&y[0]));
  if constexpr (M4) {
    if constexpr (S8 % 4 == 2) pp_slot_copies<KIND, 1>(c, bb, (uint32_t)min(u / 4 + 2, c.nslots / 2 - 1));
  } else {
    pp_slot_copies<KIND, 1>(c, slot_cur, (uint32_t)min(u / 2 + 2, c.nslots - 1));
  }
  if constexpr (SC) {
    if (S8 + 1 == 1) pp_scale_copy(c, sb_cur, min(q + 2, c.ngroups - 1));
    if (S8 + 1 == G - 1) {
      if constexpr (QA) pp_read_scales_b(c, sb_nxt, nb);
      else pp_read_scales(c, sb_nxt, na, nb);
    }
  }
  if (GR == 1) wait_vm_n(WAIT);
  pp_phase_barrier();
  // ---- C_{u+1}
  pp_mfmas<KIND, F::KSTEPS * (S8 + 1), QA, FC>(y, sa, sb, acc, sq);
  if (GR == 0) wait_vm_n(WAIT);
  pp_phase_barrier();
  if (SC && S8 + 1 == G - 1) {  // the next group's scales take over
    if constexpr (!QA) {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        sa[j][0] = na[j][0];
        sa[j][1] = na[j][1];
      }
    }
#pragma unroll
    for (int i = 0; i < 2; i++) {
      sb[i][0] = nb[i][0];
      sb[i][1] = nb[i][1];
    }
  }
}

template <int KIND, int GR, bool QA, int FC>
MX_DEV void pp_main_loop(const PPCtx& c, char* s0, char* s1, char* sb0, char* sb1, v16f (&acc)[2][4], char* asc,
                         v4i (&ld)[4]) {
  constexpr int G = PPFmt<KIND>::G;
  uint32_t sa[4][2], sb[2][2], na[4][2], nb[2][2];
  if constexpr (QA) pp_read_scales_b(c, sb0, sb);  // group 0
  else if constexpr (KIND != 4) pp_read_scales(c, sb0, sa, sb);
  if (GR == 1) raw_barrier();  // waves 4-7 start one phase late
  // Two scale groups per iteration (the group count is even), so the slot and scale buffer of every
  // step are static and the loop body has no branch: the scheduling barriers then keep every MFMA
  // in its C phase. Slot of steps u, u+1: (u/2) % 2 (2G steps cover whole pairs of slots).
  for (int q = 0; q < c.ngroups; q += 2) {
#define MX_PP(S, QQ, SC, SN)                                                                                \
  pp_step2<KIND, GR, S, QA, FC>(c, q + QQ, ((G * QQ + S) / 2) % 2 ? s1 : s0, ((G * QQ + S) / 2) % 2 ? s0 : s1, SC, SN, \
                            sa, sb, na, nb, acc, asc, ld, ((G * QQ + S) / 4) % 2 ? s1 : s0, \
                            ((G * QQ + S) / 4) % 2 ? s0 : s1)
    MX_PP(0, 0, sb0, sb1); MX_PP(2, 0, sb0, sb1);
    if constexpr (G == 8) { MX_PP(4, 0, sb0, sb1); MX_PP(6, 0, sb0, sb1); }
    MX_PP(0, 1, sb1, sb0); MX_PP(2, 1, sb1, sb0);
    if constexpr (G == 8) { MX_PP(4, 1, sb1, sb0); MX_PP(6, 1, sb1, sb0); }
#undef MX_PP
  }
  if (GR == 0) raw_barrier();  // matches the late start of waves 4-7
}

// QA: A is binary16 [M][K] and is quantised to E4M3 on load (KIND 0 only). FC: MFMA format codes of
// the byte operands (KIND 0; pp_mfmas).
template <int KIND, bool QA, int FC = 0>
__global__ __launch_bounds__(512, 1) void gemm_pp_ring_kernel(Args p) {
  using F = RingFmt<KIND>;
  using PF = PPFmt<KIND>;
  static_assert(!QA || KIND == 0, "quantise-on-load: E4M3");
  constexpr int BN = 256;
  __shared__ __attribute__((aligned(16))) char slot0[PF::SLOT2];
  __shared__ __attribute__((aligned(16))) char slot1[PF::SLOT2];
  __shared__ __attribute__((aligned(16))) char sbuf0[PF::SBUF];
  __shared__ __attribute__((aligned(16))) char sbuf1[PF::SBUF];
  __shared__ __attribute__((aligned(16))) char asc[QA ? 4 * 512 : 16];  // A scales of 4 steps (QA)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bid = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);  // each XCD takes a contiguous tile range
  // Tile order: bands of up to 8 tile rows, m fastest within a band, then n. An XCD's 32 concurrent
  // tiles then share at most 8 A panels and 4 B panels (tall grids in plain m-fastest order put 16 or
  // more A panels in one XCD's L2 at once).
  int tm, tn;
  {
    const int band = 8 * p.tiles_n, full = p.tiles_m / 8;
    const int sr = bid / band, r = bid - sr * band;
    const int rows = sr < full ? 8 : p.tiles_m - 8 * full;
    tm = 8 * sr + r % rows;
    tn = r / rows;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int rows_a = min(BM, p.M - m0), rows_b = min(BN, p.N - n0);
  // bytes per A / B row (fp16: per A row; B rows are K-rows of 2N bytes)
  const uint32_t RB = F::F16 ? 2u * (uint32_t)p.K
                     : F::F6   ? (uint32_t)p.K / 4u * 3u
                               : (uint32_t)p.K / (F::FP4 || KIND == 3 ? 2 : 1);
  const uint32_t nblk = (uint32_t)p.K / 32;
  const uint32_t RBW = KIND == 2 ? (uint32_t)p.K / 2u : KIND == 3 ? (uint32_t)p.K : RB;  // bytes per B row

  PPCtx c;
  c.wave = wave;
  c.wm = wave & 1;
  c.wn = wave >> 1;
  c.r32 = lane & 31;
  c.h = lane >> 5;
  c.nst = F::F16 ? p.K / 32 : p.K / (64 * F::KSTEPS);  // steps of 64 row bytes (FP6: 48)
  c.nslots = c.nst / 2;
  c.ngroups = c.nst / PF::G;
  {
    // copy instruction i = wave + 8k covers rows 8i..8i+7 of its operand; lane l fills physical chunk
    // l%8 of row 8i + l/8, logical chunk (l%8) ^ ((row >> 1) & 7) = (l%8) ^ ((4 (i&1) + l/16) & 7),
    // and i & 1 = wave & 1 for every copy of the wave
    const uint32_t l = (uint32_t)lane, j = l >> 3, pc = l & 7;
    const uint32_t lc = pc ^ ((4u * ((uint32_t)wave & 1u) + (j >> 1)) & 7u);
    // FP6: 96 data bytes per row, logical chunks 0..5; lanes of chunks 6, 7 re-read chunk 4, 5 of the
    // same row into unused LDS bytes (the same cache lines, so no extra HBM traffic)
    c.voff = j * RB + 16u * (F::F6 && lc >= 6u ? lc - 2u : lc);
    if constexpr (KIND == 2 || KIND == 3) c.voff_b = j * RBW + 16u * lc;
  }
  {
    // fragment chunks: row r = 128 wm + 32 j + r32 (A) or 64 wn + 32 i + r32 (B); (r >> 1) & 7 =
    // (r32 >> 1) & 7; tile j adds 4096 bytes (read offsets)
    const uint32_t r32 = (uint32_t)c.r32, h = (uint32_t)c.h, sw = (r32 >> 1) & 7u;
    const uint32_t lo = r32 * 128u + (F::F6 ? 0u : 16u * (h ^ sw));
    if constexpr (F::F6) {
#pragma unroll
      for (int hs = 0; hs < 2; hs++)
#pragma unroll
        for (int t = 0; t < 3; t++) {
          const uint32_t o = 48u * (uint32_t)hs + 24u * h + 8u * (uint32_t)t;
          c.f6o[hs][t] = 16u * ((o >> 4) ^ sw) + (o & 15u);
        }
    }
    c.fa0 = 16384u * (uint32_t)c.wm + lo;
    c.fb0 = (uint32_t)BM * 128u + 8192u * (uint32_t)c.wn + lo;
    c.sc_a = 16u * (128u * (uint32_t)c.wm + r32);
    c.sc_b = 16u * ((uint32_t)BM + 64u * (uint32_t)c.wn + r32);
  }
  // per-copy buffer resources over the copy's 8 rows, clamped to the matrix (empty past the tile)
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const int i = wave + 8 * k;
    const bool isA = i < 32;
    const int r0 = 8 * (isA ? i : i - 32), rows = isA ? rows_a : rows_b;
    const int nr = max(0, min(8, rows - r0));
    const uint32_t rb = isA ? RB : RBW;
    const uint8_t* base = (isA ? p.A + (int64_t)m0 * rb : p.B + (int64_t)n0 * rb) + (int64_t)(nr ? r0 : 0) * rb;
    c.rdata[k] = make_rsrc(base, (uint32_t)nr * rb);
    if constexpr (F::F16) {
      // B copy i - 32 of a slot: K-rows 2 (i - 32) and 2 (i - 32) + 1, 512 bytes from column n0; the
      // resource runs to the end of B. Columns past N (never stored) read the next row, or zeros
      // past the end of B: the buffer range check covers the lane offset but not the scalar offset,
      // so the slot's K-row offset goes in the lane offset (N % 8 == 0 keeps each 16-byte piece
      // inside one row, wholly in range or wholly out)
      if (!isA) {
        const uint32_t RBB = 2u * (uint32_t)p.N;
        const int64_t start = (int64_t)2 * (i - 32) * RBB + 2 * (int64_t)n0;
        c.rdata[k] = make_rsrc(p.B + start, (uint32_t)((int64_t)p.K * RBB - start));
      }
    }
  }
  if constexpr (F::F16) {
    // lane l of a B copy fills physical chunk l % 32 of K-row l / 32 of its pair, whose K-row & 3
    // is 2 (wave & 1) + l / 32 (copy index and wave have the same parity): logical chunk
    // (l % 32) ^ 4 (K-row & 3). Transposing reads: within each 16-lane group g, lane i addresses
    // K-row 8 (g / 2) + i / 4 and columns 4 (i % 4).. of the group's 16 (tile columns 16 (g % 2)..),
    // so lane l receives column l % 32 of the tile at K = 8 h + 0..3.
    const uint32_t l = (uint32_t)lane, RBB = 2u * (uint32_t)p.N;
    c.voff_b = (l >> 5) * RBB + 16u * ((l & 31u) ^ (8u * ((uint32_t)wave & 1u) + 4u * (l >> 5)));
    c.bslot = 64u * RBB;
    const uint32_t g16 = l >> 4, i16 = l & 15u, y = i16 >> 2;
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const uint32_t cc = 4u * (2u * (uint32_t)c.wn + (uint32_t)i) + 2u * (g16 & 1u) + ((i16 & 3u) >> 1);
      c.bt_off[i] = (8u * (g16 >> 1) + y) * 512u + 16u * (cc ^ (4u * y)) + 8u * (i16 & 1u);
    }
  }
  {  // scale copy of this wave: 64 rows, A rows 64w.. for w < 4, B rows 64(w-4).. after (QA: no A
     // scale plane; the A-row copies read from an empty resource and write unused zeros)
    const bool isA = wave < 4;
    const int r0 = 64 * (isA ? wave : wave - 4), rows = isA ? (QA ? 0 : rows_a) : rows_b;
    const int nr = max(0, min(64, rows - r0));
    const uint8_t* base = (isA ? p.SA + (int64_t)m0 * nblk : p.SB + (int64_t)n0 * nblk) + (int64_t)(nr ? r0 : 0) * nblk;
    c.rscale = make_rsrc(base, (uint32_t)nr * nblk);
    c.svoff = (uint32_t)lane * nblk;
  }

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;

  v4i ld[4];
  if constexpr (QA) {
    // this thread quantises row rq = tid / 2, block bq = tid % 2 of every step
    const uint32_t rq = (uint32_t)tid >> 1, bq = (uint32_t)tid & 1u, K2 = 2u * (uint32_t)p.K;
    c.ra16 = make_rsrc(p.A + (int64_t)m0 * K2, (uint32_t)rows_a * K2);
    c.qa_voff = rq * K2 + 64u * bq;
    c.qa_row = rq * 128u;
    c.qa_sw = (rq >> 1) & 7u;
    c.qa_bq = (int)bq;
    c.qa_asc_w = 2u * rq + bq;
    c.qa_asc_r = 2u * (128u * (uint32_t)c.wm + (uint32_t)c.r32) + (uint32_t)c.h;
  }

  // prologue: scale groups 0 and 1, slot 0 (steps 0, 1) and the B rows of slot 1 (its A rows are
  // queued in L_0); wait for group 0 and slot 0 (the 5 copies of group 1 and slot 1's B rows may
  // still be in flight: the first odd step waits for them). QA: steps 0 and 1 of A are quantised
  // here, and the block of step 2 loaded.
  if constexpr (!F::F16) pp_scale_copy(c, sbuf0, 0);
  if constexpr (!QA) pp_slot_copies<KIND, 0>(c, slot0, 0);
  pp_slot_copies<KIND, 1>(c, slot0, 0);
  if constexpr (!F::F16) pp_scale_copy(c, sbuf1, min(1, c.ngroups - 1));
  pp_slot_copies<KIND, 1>(c, slot1, (uint32_t)min(1, c.nslots - 1));
  if constexpr (QA) {
    v4i w0[4], w1[4];
    qa_load(c, 0, w0);
    qa_load(c, 1, w1);
    qa_store(c, 0, w0, slot0, asc);
    qa_store(c, 1, w1, slot0, asc);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    qa_load(c, min(2, c.nst - 1), ld);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the quantised steps are in LDS
  } else {
    wait_vm_n(F::F16 ? 4 : 5);  // slot 1's B rows (and group 1's scales) may still be in flight
  }
  raw_barrier();
  if (wave < 4) pp_main_loop<KIND, 0, QA, FC>(c, slot0, slot1, sbuf0, sbuf1, acc, asc, ld);
  else pp_main_loop<KIND, 1, QA, FC>(c, slot0, slot1, sbuf0, sbuf1, acc, asc, ld);
  // the last steps queued copies into the free slot: let them land, and every wave finish with the
  // slots, before they are reused for the output
  __builtin_amdgcn_s_waitcnt(0x0F70);
  raw_barrier();

  // Epilogue: as the ring's, each wave staging 64 rows x 64 columns at a time in its own 16 KB
  // quarter of a slot (rows padded by 8 bytes), then writing 16-byte row pieces.
  char* stage = ((wave & 1) ? slot1 : slot0) + (wave >> 1) * 16384;
  constexpr int WCOLS = 64, EROW = 2 * WCOLS + 8, LPR = WCOLS / 8, PIECES = 64 * LPR;
  static_assert(64 * EROW <= 16384 && PIECES % 64 == 0, "epilogue staging");
  const int r32 = c.r32, h = c.h;
  const bool rows16 = (p.N & 7) == 0;
  if (p.relu) {
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int e = 0; e < 16; e++) acc[i][j][e] = fmaxf(acc[i][j][e], 0.0f);
  }
#pragma unroll
  for (int j0 = 0; j0 < 4; j0 += 2) {
#pragma unroll
    for (int jj = 0; jj < 2; jj++)
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int qq = 0; qq < 4; qq++) {
          v4h o;
#pragma unroll
          for (int e = 0; e < 4; e++) o[e] = (_Float16)acc[i][j0 + jj][4 * qq + e];
          *reinterpret_cast<v4h*>(stage + (32 * jj + r32) * EROW + (32 * i + 8 * qq + 4 * h) * 2) = o;
        }
#pragma unroll
    for (int s0 = 0; s0 < PIECES; s0 += 64) {
      const int piece = s0 + lane, lr = piece / LPR, cp = piece % LPR;
      const char* src = stage + lr * EROW + 16 * cp;
      const v4h lo = *reinterpret_cast<const v4h*>(src), hi = *reinterpret_cast<const v4h*>(src + 8);
      const int m = m0 + 128 * c.wm + 32 * j0 + lr, n = n0 + WCOLS * c.wn + 8 * cp;
      if (m < p.M) {
        // non-temporal stores: C streams out without displacing the A and B panels that other tiles
        // still read from the L2 and the Infinity Cache
        _Float16* dst = p.C + (int64_t)m * p.N + n;
        if (n + 8 <= p.N) {
          if (rows16) {
            __builtin_nontemporal_store(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7),
                                        reinterpret_cast<v8h*>(dst));
          } else {
            __builtin_nontemporal_store(lo, reinterpret_cast<v4h*>(dst));
            __builtin_nontemporal_store(hi, reinterpret_cast<v4h*>(dst + 4));
          }
        } else if (n + 4 <= p.N) {
          __builtin_nontemporal_store(lo, reinterpret_cast<v4h*>(dst));
        }
      }
    }
  }
}

}  // namespace

namespace mx {
// Ring kernels. kind 0: E4M3 x E4M3, 1: E2M1 x E2M1, 2: E4M3 A x E2M1 B, 3: E2M1 A x E4M3 B,
// 4: fp16 x fp16 (B K x N). Requires N % 4 == 0 and K % 512 == 0 (K % 1024 == 0 for kind 1); for
// kind 4 N % 256 == 0, K % 256 == 0 and 2*K*N < 2^31, bn = 256 only. Checked by the caller.
// bn = 256, 224 or 192 (192: kinds 0 and 1). fca / fcb: the MFMA format code of the A / B operand
// where it is a byte or FP6 operand: 0 E4M3, 1 E5M2 (kinds 0, 2 (A), 3 (B)), 2 E2M3, 3 E3M2
// (kind 5); other than 0 only with 256 x 256 tiles. Returns MX_ERR_FORMAT for other combinations.
int gemm_ring_launch(int kind, int bn, int fca, int fcb, const void* A, const void* SA, const void* B,
                     const void* SB, void* C, int M, int N, int K, bool relu, hipStream_t stream) {
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
#define MX_RING(KD, WM, BNT, FA8, FB8) \
  hipLaunchKernelGGL((gemm_ring_kernel<KD, WM, BNT, FA8, FB8>), grid, block, 0, stream, a)
  const bool plain = fca == 0 && fcb == 0;  // E4M3 for every byte operand
  if (bn == 224 && plain) {
    switch (kind) {
      case 0: MX_RING(0, 4, 224, 0, 0); break;
      case 1: MX_RING(1, 4, 224, 0, 0); break;
      case 2: MX_RING(2, 4, 224, 0, 0); break;
      case 3: MX_RING(3, 4, 224, 0, 0); break;
      default: return MX_ERR_FORMAT;
    }
  } else if (bn == 192 && plain) {
    switch (kind) {
      case 0: MX_RING(0, 2, 192, 0, 0); break;
      case 1: MX_RING(1, 2, 192, 0, 0); break;
      default: return MX_ERR_FORMAT;
    }
  } else if (bn != 256) {
    return MX_ERR_FORMAT;
  } else if (kind == 5) {  // FP6 pairs: codes 2 (E2M3) / 3 (E3M2)
    if (fca == 2 && fcb == 2) MX_RING(5, 2, 256, 2, 2);
    else if (fca == 3 && fcb == 3) MX_RING(5, 2, 256, 3, 3);
    else if (fca == 2 && fcb == 3) MX_RING(5, 2, 256, 2, 3);
    else if (fca == 3 && fcb == 2) MX_RING(5, 2, 256, 3, 2);
    else return MX_ERR_FORMAT;
  } else if (!plain) {  // E5M2 (code 1) byte operands
    if (kind == 0 && fca == 1 && fcb == 1) MX_RING(0, 2, 256, 1, 1);
    else if (kind == 0 && fca == 0 && fcb == 1) MX_RING(0, 2, 256, 0, 1);
    else if (kind == 0 && fca == 1 && fcb == 0) MX_RING(0, 2, 256, 1, 0);
    else if (kind == 2 && fca == 1) MX_RING(2, 2, 256, 1, 0);
    else if (kind == 3 && fcb == 1) MX_RING(3, 2, 256, 0, 1);
    else return MX_ERR_FORMAT;
  } else {
    switch (kind) {
      case 0: MX_RING(0, 2, 256, 0, 0); break;
      case 1: MX_RING(1, 2, 256, 0, 0); break;
      case 2: MX_RING(2, 2, 256, 0, 0); break;
      case 3: MX_RING(3, 2, 256, 0, 0); break;
      case 4: MX_RING(4, 2, 256, 0, 0); break;
      default: return MX_ERR_FORMAT;
    }
  }
#undef MX_RING
  return launch_status();
}

// 8-wave ping-pong ring, 256 x 256 tiles: kind 0 (E4M3 x E4M3) or 1 (E2M1 x E2M1), K % 1024 == 0
// (an even number of scale groups), N % 4 == 0; checked by the caller.
// qa: A is binary16 [M][K], quantised to E4M3 on load (kind 0 only; SA unused).
// kind 0 (byte operands, fca / fcb the MFMA format codes of A / B: 0 = E4M3, 1 = E5M2), 1 (E2M1),
// 2 (byte A, code fca, x E2M1 B, fcb = 4), 3 (E2M1 A, fca = 4, x byte B, code fcb) or 5 (FP6, codes
// 2 = E2M3, 3 = E3M2).
int gemm_pp_ring_launch(int kind, int fca, int fcb, const void* A, const void* SA, const void* B, const void* SB,
                        void* C, int M, int N, int K, bool relu, bool qa, hipStream_t stream) {
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
  a.tiles_n = (N + 255) / 256;
  const dim3 grid((unsigned)(a.tiles_m * a.tiles_n)), block(512);
  if (kind == 0 && (fca < 0 || fca > 1 || fcb < 0 || fcb > 1)) return MX_ERR_FORMAT;
  if (kind == 5 && (fca < 2 || fca > 3 || fcb < 2 || fcb > 3)) return MX_ERR_FORMAT;
  if (kind == 2 && (fca < 0 || fca > 1 || fcb != 4)) return MX_ERR_FORMAT;
  if (kind == 3 && (fca != 4 || fcb < 0 || fcb > 1)) return MX_ERR_FORMAT;
  const int fc = kind == 0 || kind == 2 || kind == 3 || kind == 5 ? fca | (fcb << 4) : 0;
  if (qa) {
    if (kind != 0 || fc != 0) return MX_ERR_FORMAT;
    hipLaunchKernelGGL((gemm_pp_ring_kernel<0, true>), grid, block, 0, stream, a);
  } else if (kind == 0 && fc == 0x00) {
    hipLaunchKernelGGL((gemm_pp_ring_kernel<0, false, 0x00>), grid, block, 0, stream, a);
  } else if (kind == 0 && fc == 0x11) {
    hipLaunchKernelGGL((gemm_pp_ring_kernel<0, false, 0x11>), grid, block, 0, stream, a);
  } else if (kind == 0 && fc == 0x10) {
    hipLaunchKernelGGL((gemm_pp_ring_kernel<0, false, 0x10>), grid, block, 0, stream, a);
  } else if (kind == 0 && fc == 0x01) {
    hipLaunchKernelGGL((gemm_pp_ring_kernel<0, false, 0x01>), grid, block, 0, stream, a);
  } else if (kind == 1) {
    hipLaunchKernelGGL((gemm_pp_ring_kernel<1, false>), grid, block, 0, stream, a);
  } else if (kind == 2 && fc == 0x40) {
    hipLaunchKernelGGL((gemm_pp_ring_kernel<2, false, 0x40>), grid, block, 0, stream, a);
  } else if (kind == 2 && fc == 0x41) {
    hipLaunchKernelGGL((gemm_pp_ring_kernel<2, false, 0x41>), grid, block, 0, stream, a);
  } else if (kind == 3 && fc == 0x04) {
    hipLaunchKernelGGL((gemm_pp_ring_kernel<3, false, 0x04>), grid, block, 0, stream, a);
  } else if (kind == 3 && fc == 0x14) {
    hipLaunchKernelGGL((gemm_pp_ring_kernel<3, false, 0x14>), grid, block, 0, stream, a);
  } else if (kind == 4) {
    hipLaunchKernelGGL((gemm_pp_ring_kernel<4, false>), grid, block, 0, stream, a);
  } else if (kind == 5 && fc == 0x22) {
    hipLaunchKernelGGL((gemm_pp_ring_kernel<5, false, 0x22>), grid, block, 0, stream, a);
  } else if (kind == 5 && fc == 0x33) {
    hipLaunchKernelGGL((gemm_pp_ring_kernel<5, false, 0x33>), grid, block, 0, stream, a);
  } else if (kind == 5 && fc == 0x32) {
    hipLaunchKernelGGL((gemm_pp_ring_kernel<5, false, 0x32>), grid, block, 0, stream, a);
  } else if (kind == 5 && fc == 0x23) {
    hipLaunchKernelGGL((gemm_pp_ring_kernel<5, false, 0x23>), grid, block, 0, stream, a);
  } else {
    return MX_ERR_FORMAT;
  }
  return launch_status();
}
}  // namespace mx
