// api.cpp -- the C ABI of libmxgemm (declared in include/mxgemm.h): argument validation, GEMM
// plans (tile choice), device architecture check and dispatch to the kernels.
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <new>

#include "common.h"

namespace mx {
int gemm_launch(int kind, int tile_id, const void* A, const void* SA, const void* B, const void* SB, void* C, int M,
                int N, int K, bool relu, bool qa, hipStream_t stream);
int matvec_launch(int M, int N, int K, const void* x, const void* W, bool int8, const void* Ws, void* y, void* ws,
                  size_t ws_bytes, hipStream_t stream);
size_t matvec_workspace(int M, int N, int K, bool int8);
int matvec_launch_noalloc(int M, int N, int K, const void* x, const void* W, bool int8, const void* Ws, void* y,
                          hipStream_t stream);

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
}  // namespace

int check_arch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return MX_ERR_ARCH;
  }
  if (dev < kMaxDevices) {
    int v = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (v) return v == 1 ? MX_OK : MX_ERR_ARCH;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return MX_ERR_ARCH;
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? MX_OK : MX_ERR_ARCH;
}

}  // namespace mx

using namespace mx;

struct mxgemm_plan {
  int M, N, K, fa, fb, kind, tile_id;
  unsigned flags;
};

namespace {

struct TileInfo {
  int bm, bn, waves, variant;  // variant: 0 = 4 waves, 1 = 8 waves, 2 = 8-wave ping-pong (MX only),
                               // 3 = 4-stage LDS ring (MX formats; fp16 on 256x256),
                               // 4 = 8-wave ping-pong ring (E4M3, E2M1, fp16)
  int eff[3];                  // measured relative efficiency per kind (E4M3, E2M1, F16), percent
};
// Tile ids understood by gemm_launch. The efficiencies rank the tiles (MI355X measurements at the
// prefill / large GEMM shapes; 256x256 ping-pong spills registers and is ranked low; the 256x224
// ring runs the prefill shape in two whole rounds but no faster than the 256x256 ring's 1.75, so it
// is ranked below it; a partial last round runs faster per tile than a full one, the chip being
// shared-resource bound). The 256x192 ring wins where it makes whole rounds and 256x256 does not
// (M=2048, N=12288: 95 against 101 us). The 8-wave ping-pong GEMM with 128-byte stage rows (tile
// 11, where K % 1024 == 0) is the fastest tile at every shape measured, also where 256x192 ring
// tiles make whole rounds and its 256x256 tiles do not (E4M3, K=4096: M=2048 N=12288 92.3 against
// 97.9 us, M=2048 N=4096 37.9 against 38.7 us, M=512 N=8192 K=8192 67.0 against 67.0 us; MXFP8
// prefill 97.1 against 109.7-126.8 us for the ring tiles; MXFP4 4096 x 8192 x 8192 128.8 against
// 138.7-167.5 us). fp16 on tile 11 (K % 512 == 0): 4096^3 109.9 against 114.3 us on the ring,
// 2048 x 14336 x 4096 201.1 against 208.6 us, 8192^3 803 against 1199 us.
constexpr TileInfo kTiles[] = {
    {256, 256, 4, 0, {85, 85, 90}}, {256, 224, 4, 0, {80, 75, 55}}, {128, 128, 4, 0, {50, 45, 50}},
    {64, 64, 4, 0, {25, 25, 25}},   {256, 256, 8, 1, {90, 100, 100}}, {256, 224, 8, 1, {88, 95, 60}},
    {256, 256, 8, 2, {60, 60, 99}}, {256, 224, 8, 2, {100, 95, 60}}, {256, 256, 4, 3, {200, 200, 200}},
    {256, 224, 4, 3, {170, 160, 1}}, {256, 192, 4, 3, {170, 160, 1}}, {256, 256, 8, 4, {240, 240, 240}}};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);
constexpr int kRingTile = 8, kRingTile224 = 9, kRingTile192 = 10, kPPRingTile = 11;
constexpr int kCUs = 256;

// Whether the ping-pong ring (tile 11) runs fp16 x fp16: K a multiple of 512 (whole pairs of 4-step
// scale-less groups of 32 K, and at least the 16 steps of the smallest MX case), B rows (2N bytes)
// in whole 16-byte chunks, byte offsets into B within 31 bits.
bool pp16_ok(int N, int K) { return K % 512 == 0 && N % 8 == 0 && 2 * (int64_t)K * N < ((int64_t)1 << 31); }

// Whether ring tile `tile` (8: 256x256, 9: 256x224) runs the ring kernel for this problem; the
// fp16 ring exists for 256x256 only.
bool ring_ok(int kind, int N, int K, int tile) {
  if (kind == 2)
    return tile == 8 && N % 256 == 0 && K % 256 == 0 && 2 * (int64_t)K * N < ((int64_t)1 << 31);
  if (tile == kRingTile192 && kind >= 3) return false;
  return N % 4 == 0 && ((kind == 0 && K % 512 == 0) || (kind == 1 && K % 1024 == 0));
}

int choose_tile(int kind, int M, int N, int K) {
  if (const char* env = std::getenv("MXGEMM_TILE")) {
    int t = std::atoi(env);
    // pairs other than the three plain ones run on the ring (256x224 for E4M3 / E2M1 mixes), or on
    // the ping-pong ring (tile 11) for E5M2 with E5M2 / E4M3 and the FP6 pairs
    if (t >= 0 && t < kNumTiles) {
      if (kind >= 3 && t == kPPRingTile) return t;
      return kind >= 3 ? (t == kRingTile224 && kind <= 4 ? t : kRingTile) : t;
    }
  }
  // the mixed, E5M2 and FP6 pairs: the ping-pong ring where it applies, else the 4-stage ring
  if (kind >= 3) return K % 1024 == 0 && N % 4 == 0 ? kPPRingTile : kRingTile;
  int best = 0;
  double best_cost = 1e300;
  for (int t = 0; t < kNumTiles; t++) {
    if ((t == kRingTile || t == kRingTile224 || t == kRingTile192) && !ring_ok(kind, N, K, t)) continue;
    if (t == kPPRingTile && !((kind <= 1 && K % 1024 == 0 && N % 4 == 0) || (kind == 2 && pp16_ok(N, K)))) continue;
    const int64_t tiles = (int64_t)((M + kTiles[t].bm - 1) / kTiles[t].bm) * ((N + kTiles[t].bn - 1) / kTiles[t].bn);
    const int64_t waves = (tiles + kCUs - 1) / kCUs;
    const double cost = (double)waves * kTiles[t].bm * kTiles[t].bn * 100.0 / kTiles[t].eff[kind];
    if (cost < best_cost) {
      best_cost = cost;
      best = t;
    }
  }
  return best;
}

}  // namespace

extern "C" {

const char* mx_strerror(mx_status s) {
  switch (s) {
    case MX_OK: return "ok";
    case MX_ERR_NULL: return "a required pointer is NULL";
    case MX_ERR_SHAPE: return "unsupported or invalid dimensions";
    case MX_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case MX_ERR_FORMAT: return "unsupported format or format pair";
    case MX_ERR_ARCH: return "current device is not gfx950 (or no device)";
    case MX_ERR_LAUNCH: return "kernel launch failed";
    case MX_ERR_NOMEM: return "host allocation failed";
    case MX_ERR_SCRATCH: return "the shape needs more workspace than the library's static scratch array holds";
    default: return "unknown status";
  }
}

int mx_version(void) { return 100; }

int mxgemm_create(mxgemm_t* out, int M, int N, int K, int fa, int fb, unsigned flags) {
  if (!out) return MX_ERR_NULL;
  *out = nullptr;
  if (flags & ~(unsigned)(MXGEMM_RELU | MXGEMM_QUANT_A)) return MX_ERR_FORMAT;
  const bool qa = (flags & MXGEMM_QUANT_A) != 0u;
  if (qa && !(fa == MX_E4M3 && fb == MX_E4M3)) return MX_ERR_FORMAT;
  int kind;
  if (fa == MX_E4M3 && fb == MX_E4M3) kind = 0;
  else if (fa == MX_E2M1 && fb == MX_E2M1) kind = 1;
  else if (fa == MX_F16 && fb == MX_F16) kind = 2;
  else if (fa == MX_E4M3 && fb == MX_E2M1) kind = 3;
  else if (fa == MX_E2M1 && fb == MX_E4M3) kind = 4;
  else if (fa == MX_E5M2 && fb == MX_E5M2) kind = 5;
  else if (fa == MX_E4M3 && fb == MX_E5M2) kind = 6;
  else if (fa == MX_E5M2 && fb == MX_E4M3) kind = 7;
  else if (fa == MX_E5M2 && fb == MX_E2M1) kind = 8;
  else if (fa == MX_E2M1 && fb == MX_E5M2) kind = 9;
  else if (fa == MX_E2M3 && fb == MX_E2M3) kind = 10;
  else if (fa == MX_E3M2 && fb == MX_E3M2) kind = 11;
  else if (fa == MX_E2M3 && fb == MX_E3M2) kind = 12;
  else if (fa == MX_E3M2 && fb == MX_E2M3) kind = 13;
  else return MX_ERR_FORMAT;
  if (M < 1 || N < 1 || K < 32 || M > MX_MAX_DIM || N > MX_MAX_DIM || K > MX_MAX_DIM) return MX_ERR_SHAPE;
  if (kind != 2 && K % 32) return MX_ERR_SHAPE;
  if (kind == 2 && (K % 8 || N % 8)) return MX_ERR_SHAPE;
  if (kind >= 3 && (K % 512 || N % 4)) return MX_ERR_SHAPE;  // mixed, E5M2 and FP6 pairs: the ring kernel only
  if (qa && (K % 1024 || N % 4)) return MX_ERR_SHAPE;         // quantise-on-load: the ping-pong kernel only
  mxgemm_plan* p = new (std::nothrow) mxgemm_plan{M, N, K, fa, fb, kind, qa ? kPPRingTile : choose_tile(kind, M, N, K),
                                                  flags};
  if (!p) return MX_ERR_NOMEM;
  *out = p;
  return MX_OK;
}

int mxgemm_destroy(mxgemm_t p) {
  delete p;
  return MX_OK;
}

int mxgemm_plan_info(mxgemm_t p, int* tile_m, int* tile_n, int* tile_k, int* variant) {
  if (!p || !tile_m || !tile_n || !tile_k || !variant) return MX_ERR_NULL;
  const TileInfo& t = kTiles[p->tile_id];
  *tile_m = t.bm;
  *tile_n = t.bn;
  *tile_k = p->kind == 0 ? 128 : (p->kind == 1 ? 256 : 64);  // mixed pairs: 64 (the ring's stage)
  if (p->tile_id == kPPRingTile && p->kind != 2 &&
      p->K % 1024 == 0 && p->N % 4 == 0) {
    *tile_k = p->kind == 1 ? 128 : 64;  // the 8-wave ping-pong ring
    *variant = 4;
    return MX_OK;
  }
  if (p->tile_id == kPPRingTile && p->kind == 2 && pp16_ok(p->N, p->K)) {
    *tile_k = 32;  // fp16 on the ping-pong ring: 64-byte steps of 32 K
    *variant = 4;
    return MX_OK;
  }
  if (p->tile_id == kRingTile || p->tile_id == kRingTile224 || p->tile_id == kRingTile192 || p->tile_id == kPPRingTile) {
    // the ring, or the 8-wave kernel where it does not apply (256 x 256 in place of 256 x 192); tile 11
    // where the ping-pong ring does not apply falls back as tile 8 does
    const int rt = p->tile_id == kPPRingTile ? kRingTile : p->tile_id;
    const bool ring = p->kind >= 3 || ring_ok(p->kind, p->N, p->K, rt);
    if (!ring && p->tile_id == kRingTile192) *tile_n = 256;
    *tile_k = ring ? (p->kind == 1 ? 128 : (p->kind == 2 ? 32 : 64)) : *tile_k;
    *variant = ring ? 3 : 1;
    return MX_OK;
  }
  // the ping-pong kernel needs whole stages and dword-aligned scale rows; otherwise 8 waves run
  const bool pp_ok = p->kind != 2 && (p->kind == 0 ? p->K % 128 == 0 : p->K % 256 == 0) && (p->K / 32) % 4 == 0;
  *variant = (t.variant == 2 && !pp_ok) ? 1 : (t.variant == 2 && p->kind == 2 ? 1 : t.variant);
  return MX_OK;
}

int mxgemm_run(mxgemm_t p, const void* A, const void* SA, const void* B, const void* SB, void* C, void* stream) {
  if (!p || !A || !B || !C) return MX_ERR_NULL;
  const bool qa = (p->flags & MXGEMM_QUANT_A) != 0u;  // A is binary16, SA is not used
  if (p->kind != 2 && ((!SA && !qa) || !SB)) return MX_ERR_NULL;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return MX_ERR_ALIGN;
  if (p->kind != 2 && ((!qa && !aligned16(SA)) || !aligned16(SB))) return MX_ERR_ALIGN;
  if (int a = check_arch()) return a;
  return sync_check(gemm_launch(p->kind, p->tile_id, A, SA, B, SB, C, p->M, p->N, p->K,
                                (p->flags & MXGEMM_RELU) != 0u, qa, as_stream(stream)),
                    as_stream(stream));
}

static int matvec_shape(int M, int N, int K, int fw) {
  if (fw != MX_INT8 && fw != MX_INT4) return MX_ERR_FORMAT;
  if (M < 1 || M > 256 || N < 1 || N > MX_MAX_DIM || K < 32 || K > MX_MAX_DIM || K % 32) return MX_ERR_SHAPE;
  if (fw == MX_INT8 ? (N % 16) : (N % 32)) return MX_ERR_SHAPE;
  return MX_OK;
}

size_t mxmatvec_workspace_size(int M, int N, int K, int fw) {
  if (matvec_shape(M, N, K, fw)) return 0;
  return matvec_workspace(M, N, K, fw == MX_INT8);
}

int mxmatvec_run(int M, int N, int K, const void* x, const void* W, int fw, const void* Ws, void* y, void* workspace,
                 size_t workspace_bytes, void* stream) {
  if (!x || !W || !Ws || !y) return MX_ERR_NULL;
  if (int s = matvec_shape(M, N, K, fw)) return s;
  if (!aligned16(x) || !aligned16(W) || !aligned16(Ws) || !aligned16(y)) return MX_ERR_ALIGN;
  if (workspace && !aligned16(workspace)) return MX_ERR_ALIGN;
  if (int a = check_arch()) return a;
  return sync_check(matvec_launch(M, N, K, x, W, fw == MX_INT8, Ws, y, workspace, workspace ? workspace_bytes : 0,
                                  as_stream(stream)),
                    as_stream(stream));
}

int mxmatvec_run_noalloc(int M, int N, int K, const void* x, const void* W, int fw, const void* Ws, void* y,
                         void* stream) {
  if (!x || !W || !Ws || !y) return MX_ERR_NULL;
  if (int s = matvec_shape(M, N, K, fw)) return s;
  if (!aligned16(x) || !aligned16(W) || !aligned16(Ws) || !aligned16(y)) return MX_ERR_ALIGN;
  if (matvec_workspace(M, N, K, fw == MX_INT8) > MXMATVEC_SCRATCH_BYTES) return MX_ERR_SCRATCH;
  if (int a = check_arch()) return a;
  return sync_check(matvec_launch_noalloc(M, N, K, x, W, fw == MX_INT8, Ws, y, as_stream(stream)), as_stream(stream));
}

}  // extern "C"
