// matvec.hip -- int8 / int4 dequant matvec for decode (M <= 8 activation rows), no MFMA.
//
//   y[m,n] = sum_b Ws[b,n] * sum_{k in block b} x[m,k] * q[k,n]     (32-row blocks b)
//
// the per-block fp16-scale form of "TensorOps ... notes", section "Kernel-phase findings"
// (revised strategy), with the int4 packing of section "VALIDATED ON M4 MAX", fact 5.
//
// The weight matrix is the only large operand, so the kernel is organised around streaming it
// exactly once from HBM:
//  - A workgroup owns a strip of TW = 64 columns over the whole of K, so every output is finished
//    by one workgroup (no partial sums leave the chip, no second pass, no scratch memory).
//  - Lane l of a wave owns 8 adjacent columns (column group l%8) and one "row phase" (l/8); the
//    8 waves give 64 row phases, and phase p walks the 8-row chunks p, p+64, p+128, ... of K.
//    One load instruction of a wave fetches 8 rows x 64 contiguous bytes (int8).
//  - Weights are turned into exact fp16 pairs (q[k,n], q[k+1,n]) with a byte permute and one
//    packed fp16 subtract (1024+128+q in the fp16 mantissa, minus 1152); the MACs are
//    v_dot2_f32_f16 with fp32 accumulation; the fp16 block scale multiplies each 8-row partial.
//  - Row phases of a wave are summed with xor shuffles (lane bits 3..5), then the 8 waves' sums
//    in LDS; the fp32 result is rounded once to fp16.
#include "codec_math.h"

using namespace mx;

namespace {

typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kCG = 8;                 // column groups per wave
constexpr int kCPL = 8;                // columns per lane
constexpr int kTW = kCG * kCPL;        // columns per workgroup
constexpr int kPhases = kWaves * (64 / kCG);

MX_DEV v2h as_v2h(uint32_t u) { return __builtin_bit_cast(v2h, u); }

// fp16 pairs (q[2p][c], q[2p+1][c]) for the 4 columns held in one dword of two consecutive rows.
// ua/ub: offset-binary bytes (q + 128) of rows 2p and 2p+1. Output w[j] for column j of the dword.
MX_DEV void pairs_from_bytes(uint32_t ua, uint32_t ub, uint32_t bias_bits, v2h (&w)[4]) {
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const uint32_t sel = (uint32_t)j | (0x0Cu << 8) | ((uint32_t)(4 + j) << 16) | (0x0Cu << 24);
    const uint32_t pr = __builtin_amdgcn_perm(ub, ua, sel) | 0x64006400u;
    w[j] = as_v2h(pr) - as_v2h(bias_bits);
  }
}

template <int M, bool I8>
__global__ __launch_bounds__(kThreads) void matvec_kernel(const _Float16* __restrict__ x, const uint8_t* __restrict__ W,
                                                          const _Float16* __restrict__ Ws, _Float16* __restrict__ y,
                                                          int N, int K) {
  __shared__ float red[kWaves][M][kTW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cg = lane % kCG, phase = wave * (64 / kCG) + lane / kCG;

  int bid = blockIdx.x;
  const int nwg = gridDim.x;
  if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);  // neighbouring strips share an XCD
  const int n0 = bid * kTW, nc = n0 + cg * kCPL;                   // first column of this lane
  const bool active = nc < N;

  float acc[M][kCPL];
#pragma unroll
  for (int m = 0; m < M; m++)
#pragma unroll
    for (int c = 0; c < kCPL; c++) acc[m][c] = 0.0f;

  // int8: 1024+128 = 1152 (0x6480); int4: 1024+8 = 1032 (0x6408)
  const uint32_t bias_bits = I8 ? 0x64806480u : 0x64086408u;
  const int nchunks = K / 8;
  if (active) {
    for (int ch = phase; ch < nchunks; ch += kPhases) {
      const int k0 = ch * 8;
      // 8 rows x 8 columns of weights as fp16 pairs: wp[c][p] = (q[k0+2p][c], q[k0+2p+1][c])
      v2h wp[kCPL][4];
      if constexpr (I8) {
        uint2 raw[8];
#pragma unroll
        for (int r = 0; r < 8; r++) raw[r] = *reinterpret_cast<const uint2*>(W + (int64_t)(k0 + r) * N + nc);
#pragma unroll
        for (int p = 0; p < 4; p++) {
          v2h t0[4], t1[4];
          pairs_from_bytes(raw[2 * p].x ^ 0x80808080u, raw[2 * p + 1].x ^ 0x80808080u, bias_bits, t0);
          pairs_from_bytes(raw[2 * p].y ^ 0x80808080u, raw[2 * p + 1].y ^ 0x80808080u, bias_bits, t1);
#pragma unroll
          for (int j = 0; j < 4; j++) {
            wp[j][p] = t0[j];
            wp[4 + j][p] = t1[j];
          }
        }
      } else {
        uint32_t raw[8];
#pragma unroll
        for (int r = 0; r < 8; r++) raw[r] = *reinterpret_cast<const uint32_t*>(W + ((int64_t)(k0 + r) * N + nc) / 2);
#pragma unroll
        for (int p = 0; p < 4; p++) {
          // even columns (low nibbles) and odd columns (high nibbles) spread into bytes
          const uint32_t ae = (raw[2 * p] & 0x0F0F0F0Fu) ^ 0x08080808u, ao = ((raw[2 * p] >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;
          const uint32_t be = (raw[2 * p + 1] & 0x0F0F0F0Fu) ^ 0x08080808u,
                         bo = ((raw[2 * p + 1] >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;
          v2h te[4], to[4];
          pairs_from_bytes(ae, be, bias_bits, te);
          pairs_from_bytes(ao, bo, bias_bits, to);
#pragma unroll
          for (int j = 0; j < 4; j++) {
            wp[2 * j][p] = te[j];
            wp[2 * j + 1][p] = to[j];
          }
        }
      }
      // block scales of these 8 columns
      const uint4 sraw = *reinterpret_cast<const uint4*>(Ws + (int64_t)(k0 / 32) * N + nc);
      float s[kCPL];
      {
        const uint32_t sv[4] = {sraw.x, sraw.y, sraw.z, sraw.w};
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const v2h h = as_v2h(sv[j]);
          s[2 * j] = (float)h[0];
          s[2 * j + 1] = (float)h[1];
        }
      }
#pragma unroll
      for (int m = 0; m < M; m++) {
        const uint4 xr = *reinterpret_cast<const uint4*>(x + (int64_t)m * K + k0);
        const v2h xp[4] = {as_v2h(xr.x), as_v2h(xr.y), as_v2h(xr.z), as_v2h(xr.w)};
#pragma unroll
        for (int c = 0; c < kCPL; c++) {
          float t = 0.0f;
#pragma unroll
          for (int p = 0; p < 4; p++) t = __builtin_amdgcn_fdot2(xp[p], wp[c][p], t, false);
          acc[m][c] = __builtin_fmaf(s[c], t, acc[m][c]);
        }
      }
    }
  }

  // Sum the 8 row phases of this wave (lane bits 3..5), then the waves through LDS.
#pragma unroll
  for (int m = 0; m < M; m++)
#pragma unroll
    for (int c = 0; c < kCPL; c++) {
      float v = acc[m][c];
      v += __shfl_xor(v, 8);
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      acc[m][c] = v;
    }
  if (lane < kCG) {
#pragma unroll
    for (int m = 0; m < M; m++)
#pragma unroll
      for (int c = 0; c < kCPL; c++) red[wave][m][cg * kCPL + c] = acc[m][c];
  }
  __syncthreads();
  for (int o = tid; o < M * kTW; o += kThreads) {
    const int m = o / kTW, col = o % kTW;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; w++) v += red[w][m][col];
    if (n0 + col < N) y[(int64_t)m * N + n0 + col] = (_Float16)v;
  }
}

template <bool I8>
int launch_m(int M, int N, int K, const void* x, const void* W, const void* Ws, void* y, hipStream_t st) {
  const dim3 grid((unsigned)((N + kTW - 1) / kTW)), block(kThreads);
  auto xx = (const _Float16*)x;
  auto ww = (const uint8_t*)W;
  auto ss = (const _Float16*)Ws;
  auto yy = (_Float16*)y;
  switch (M) {
    case 1: hipLaunchKernelGGL((matvec_kernel<1, I8>), grid, block, 0, st, xx, ww, ss, yy, N, K); break;
    case 2: hipLaunchKernelGGL((matvec_kernel<2, I8>), grid, block, 0, st, xx, ww, ss, yy, N, K); break;
    case 3: hipLaunchKernelGGL((matvec_kernel<3, I8>), grid, block, 0, st, xx, ww, ss, yy, N, K); break;
    case 4: hipLaunchKernelGGL((matvec_kernel<4, I8>), grid, block, 0, st, xx, ww, ss, yy, N, K); break;
    case 5: hipLaunchKernelGGL((matvec_kernel<5, I8>), grid, block, 0, st, xx, ww, ss, yy, N, K); break;
    case 6: hipLaunchKernelGGL((matvec_kernel<6, I8>), grid, block, 0, st, xx, ww, ss, yy, N, K); break;
    case 7: hipLaunchKernelGGL((matvec_kernel<7, I8>), grid, block, 0, st, xx, ww, ss, yy, N, K); break;
    case 8: hipLaunchKernelGGL((matvec_kernel<8, I8>), grid, block, 0, st, xx, ww, ss, yy, N, K); break;
    default: return MX_ERR_SHAPE;
  }
  return launch_status();
}

}  // namespace

namespace mx {
int matvec_launch(int M, int N, int K, const void* x, const void* W, bool int8, const void* Ws, void* y,
                  hipStream_t stream) {
  return int8 ? launch_m<true>(M, N, K, x, W, Ws, y, stream) : launch_m<false>(M, N, K, x, W, Ws, y, stream);
}
}  // namespace mx
