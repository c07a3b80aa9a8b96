/*
 * mxgemm.h -- C ABI of libmxgemm.so: block-scaled (MX) quantized GEMM, fp16 GEMM, int8/int4
 * dequant matvec and the MX/int codecs, for AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 *  - Every function returns an mx_status; 0 is success. Arguments are validated before any work
 *    is queued, and nothing is written when validation fails.
 *  - Device pointers are owned by the caller (allocated with hipMalloc or by a framework); the
 *    library never allocates, frees or retains them. Host pointers likewise.
 *  - `stream` is a hipStream_t passed as an opaque pointer (NULL = the default stream). GPU entry
 *    points only enqueue work on that stream and return; they never synchronise. Calls on
 *    different streams may run concurrently.
 *  - Debugging: with the environment variable MX_SYNC_CHECK set (to anything but "0"; read at
 *    every call), a GPU entry point that queued work waits for its stream before returning and
 *    returns MX_ERR_LAUNCH when the stream reports an error, so an asynchronous fault is reported
 *    by the call that caused it.
 *  - Device pointers must be 16-byte aligned. Matrices are dense and row-major with the leading
 *    dimension equal to the row length given below.
 *  - A GPU entry point called on a device that is not gfx950 returns MX_ERR_ARCH.
 *
 * Formats (the pages name the types, the OCP Microscaling v1.0 formats give their bits):
 *  - MX_E4M3: FP8 E4M3 "FN" (bias 7, S.1111.111 = NaN, no Inf, max 448), one byte per element.
 *  - MX_E5M2: FP8 E5M2 (bias 15, S.11111.00 = Inf, S.11111.xx = NaN, max 57344), one byte per
 *    element (the pages' fp8 / "MX scaling formats", TensorOps notes, quantized dtype matrix).
 *  - MX_E2M3 / MX_E3M2: FP6 (bias 1, max 7.5 / bias 3, max 28; no Inf or NaN), four elements per
 *    three bytes: element j in bits 6j..6j+5 of the row read as a little-endian bit stream.
 *  - MX_E2M1: FP4 E2M1 (bias 1, +-{0,.5,1,1.5,2,3,4,6}), two elements per byte, the element with
 *    the even index in the low nibble.
 *  - Scales of MX operands: E8M0 bytes, value 2^(e-127), 0xFF = NaN; one scale per 32
 *    consecutive elements along K ("Scale planes: one MTLTensor = data + scales" and the
 *    auxiliary-plane blockFactors {32,1} of the WWDC26 session 330 summary).
 *  - MX_F16: IEEE binary16. MX_INT8: two's-complement bytes. MX_INT4: two's-complement nibbles,
 *    packed two per byte along the C-order linear index, the even index in the low nibble
 *    ("TensorOps ... notes", section "VALIDATED ON M4 MAX", fact 5).
 */
#ifndef MXGEMM_H
#define MXGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MX_OK = 0,
  MX_ERR_NULL = -1,    /* a required pointer is NULL */
  MX_ERR_SHAPE = -2,   /* a dimension is out of range or violates a divisibility rule */
  MX_ERR_ALIGN = -3,   /* a device pointer is not 16-byte aligned */
  MX_ERR_FORMAT = -4,  /* unsupported format or format pair */
  MX_ERR_ARCH = -5,    /* the current device is not gfx950, or no device is present */
  MX_ERR_LAUNCH = -6,  /* the HIP runtime reported an error when queueing a kernel (or, with
                          MX_SYNC_CHECK, when the stream ran it) */
  MX_ERR_NOMEM = -7,   /* host allocation of a plan failed */
  MX_ERR_SCRATCH = -8  /* mxmatvec_run_noalloc: the shape needs more than MXMATVEC_SCRATCH_BYTES */
} mx_status;

/* MX_E8M0 names the scale format; it is accepted only by mx_decode_host. */
typedef enum { MX_E4M3 = 0, MX_E5M2 = 1, MX_E2M3 = 2, MX_E3M2 = 3, MX_E2M1 = 4, MX_E8M0 = 8, MX_F16 = 16, MX_INT8 = 32, MX_INT4 = 33 } mx_format;

/* Largest accepted dimension of any matrix (rows or columns). */
#define MX_MAX_DIM (1 << 20)

/* Human-readable name of a status code (static storage, never NULL; unknown codes are named as
 * such). */
const char* mx_strerror(mx_status status);

/* Library version as 10000*major + 100*minor + patch. */
int mx_version(void);

/* ------------------------------------------------------------------------------------------ */
/* GEMM plans.                                                                                  */
/* ------------------------------------------------------------------------------------------ */

typedef struct mxgemm_plan* mxgemm_t;

/* mxgemm_create flag: epilogue ReLU, C = max(A*B, 0) elementwise before the fp16 store, with
 * IEEE maxNum semantics (a NaN product gives 0). This is the postfix activation of the "Running
 * inline ML operations in a shader with Metal 4" sample, section "Combine an element-wise
 * function" (there applied with max(value, 0) to the product tile in registers). */
#define MXGEMM_RELU 1u

/* mxgemm_create flag: the A operand is given unquantised, as binary16 [M][K] (row-major), and is
 * quantised to E4M3 with E8M0 scales per 32 along K inside the GEMM, as the kernel loads its tiles,
 * with exactly the codes and scales mx_pack_run(MX_E4M3) gives for the same values (held in fp32):
 * C equals the product of mx_pack_run's A with B. This is the quantise-on-load of prefill
 * activations, which the pages' quantized matmul takes already quantized ("TensorOps ... notes",
 * section "Why this matters here": prefill is the compute-bound stage; scale rule of mx_pack_run).
 * Needs fa == fb == MX_E4M3 (else MX_ERR_FORMAT), K % 1024 == 0 and N % 4 == 0 (else MX_ERR_SHAPE);
 * mxgemm_run then takes SA = NULL (ignored). */
#define MXGEMM_QUANT_A 2u

/*
 * mxgemm_create -- validate a GEMM problem C[M,N] = A[M,K] * B[K,N] and choose its kernel.
 *
 * Operation ("TensorOps ... notes", sections "Scale planes" and "Kernel-phase findings"; WWDC26
 * session 330 summary, sections on the MXFP8 tensor type and the quantized matmul2d):
 *   C[m,n] = sum_k (dec(A[m,k]) * 2^(SA[m,k/32]-127)) * (dec(B[k,n]) * 2^(SB[n,k/32]-127)),
 * accumulated in fp32 and written once as fp16 (rounded to nearest even). C is overwritten
 * (C = A*B, not C += A*B). For fa == fb == MX_F16 there are no scales: C = A*B in fp32, fp16 out.
 *
 * Supported pairs: (MX_E4M3, MX_E4M3), (MX_E2M1, MX_E2M1), (MX_F16, MX_F16), and the mixed MX pairs
 * (MX_E4M3, MX_E2M1), (MX_E2M1, MX_E4M3) (A and B each in its own format, scales as above; the
 * scaled MFMA takes each operand's format separately), and every pair with an MX_E5M2 operand:
 * (MX_E5M2, MX_E5M2), (MX_E4M3, MX_E5M2), (MX_E5M2, MX_E4M3), (MX_E5M2, MX_E2M1),
 * (MX_E2M1, MX_E5M2), and the four FP6 pairs (MX_E2M3, MX_E2M3), (MX_E3M2, MX_E3M2),
 * (MX_E2M3, MX_E3M2), (MX_E3M2, MX_E2M3) (the pages' "MX scaling formats", TensorOps notes,
 * quantized dtype matrix). All pairs other than the three plain ones need K % 512 == 0 and
 * N % 4 == 0, else MX_ERR_SHAPE; FP6 with any other format is MX_ERR_FORMAT.
 * Shape rules: 1 <= M, N <= MX_MAX_DIM; 32 <= K <= MX_MAX_DIM; MX formats need K % 32 == 0;
 * MX_F16 needs K % 8 == 0 and N % 8 == 0.
 * `flags` is 0 or a combination of MXGEMM_RELU and MXGEMM_QUANT_A (other bits: MX_ERR_FORMAT).
 * Host only: queues no GPU work. *out
 * receives a plan that holds host metadata only; release it with mxgemm_destroy. A plan may be
 * used from several threads and streams at once.
 */
int mxgemm_create(mxgemm_t* out, int M, int N, int K, int fa, int fb, unsigned flags);

/*
 * mxgemm_run -- queue the GEMM of plan p on `stream`.
 *
 * Layouts (all device pointers, 16-byte aligned):
 *   MX:  A  codes [M][K] (E4M3, E5M2), [M][3K/4] (E2M3, E3M2: 6-bit fields, little-endian bit
 *           stream) or [M][K/2] (E2M1), K contiguous;
 *        SA E8M0 [M][K/32];
 *        B  codes stored K-contiguous, i.e. [N][K], [N][3K/4] or [N][K/2] by format: the scaled
 *           right operand is the transposed one ("Kernel-phase findings", fact 2);
 *        SB E8M0 [N][K/32];
 *   F16: A binary16 [M][K]; B binary16 [K][N] (row-major K x N); SA = SB = NULL.
 *   C:   binary16 [M][N].
 * Errors: MX_ERR_NULL (p, A, B, C, or a scale pointer of an MX plan), MX_ERR_ALIGN, MX_ERR_ARCH,
 * MX_ERR_LAUNCH. Non-finite inputs propagate: a NaN code or a 0xFF scale makes every output it
 * contributes to NaN. E5M2 Inf codes (S.11111.00) are infinities and follow IEEE arithmetic: an
 * output with one infinite term is that infinity, +Inf and -Inf terms together give NaN, and an
 * infinity times a zero element gives NaN (the products are formed exactly and summed in fp32).
 */
int mxgemm_run(mxgemm_t p, const void* A, const void* SA, const void* B, const void* SB, void* C,
               void* stream);

/* mxgemm_destroy -- release a plan (NULL is accepted and ignored). */
int mxgemm_destroy(mxgemm_t p);

/* Kernel chosen by a plan (for reports): output tile rows and columns, K elements per pipeline
 * stage, and the kernel variant (0: 4 waves, 1: 8 waves, 2: 8-wave ping-pong schedule, 3: 4-stage
 * LDS ring of 64-byte K stages, for MX formats with N % 4 == 0 and K % 512 == 0 (E4M3) or
 * K % 1024 == 0 (E2M1), and for fp16 with N % 256 == 0, K % 256 == 0 on 256x256 tiles; 4: 8-wave
 * ping-pong ring of 128-byte stage rows (FP6: 96) on 256x256 tiles, for every MX pair where
 * K % 1024 == 0 and N % 4 == 0 (the E2M1 operand of a mix with a byte format staged four K-steps
 * at a time), for fp16 where K % 512 == 0 and N % 8 == 0, and for MXGEMM_QUANT_A). The environment
 * variable MXGEMM_TILE (a tile id 0..11; 8, 9 and 10 are the 4-stage ring with 256x256, 256x224
 * and 256x192 tiles where it applies, else an 8-wave kernel: 256x256 for 8 and 10, 256x224 for 9;
 * 11 is the ping-pong ring where it applies, else as 8), read at mxgemm_create, overrides the
 * choice. */
int mxgemm_plan_info(mxgemm_t p, int* tile_m, int* tile_n, int* tile_k, int* variant);

/* ------------------------------------------------------------------------------------------ */
/* Dequant matvec for decode.                                                                   */
/* ------------------------------------------------------------------------------------------ */

/*
 * mxmatvec_run -- y[m,n] = sum_b Ws[b,n] * sum_{k=32b}^{32b+31} x[m,k] * q[k,n], accumulated in
 * fp32, y written as fp16. This is the per-32-row block form with arbitrary fp16 scales
 * ("TensorOps ... notes", section "Kernel-phase findings", revised kernel strategy; int4 packing
 * from section "VALIDATED ON M4 MAX", fact 5).
 *
 *   x  binary16 [M][K]      W int8 [K][N]  (fw = MX_INT8)  or packed int4 [K][N/2] (fw = MX_INT4)
 *   Ws binary16 [K/32][N]   y binary16 [M][N]
 * Shape rules: 1 <= M <= 256; K % 32 == 0, 32 <= K <= MX_MAX_DIM; 1 <= N <= MX_MAX_DIM;
 * N % 16 == 0 (int8) or N % 32 == 0 (int4). Device pointers, 16-byte aligned.
 * M <= 8 is the decode matvec; 9 <= M <= 256 (the W8A16 / W4A16 prefill-like GEMM with the same
 * arbitrary fp16 block scales, TensorOps notes, section "Kernel-phase findings") runs a small-M
 * GEMM kernel: each block product is still formed exactly in fp32 and scaled once by its fp16
 * block scale.
 *
 * Workspace (an addition to the call the pages' operation needs: workspace = NULL gives exactly
 * that call). The fastest kernels split K across workgroups: their fp32 partial sums and one counter
 * per column strip (M <= 8) or per tile (M > 8) live in a caller-owned device buffer of
 * mxmatvec_workspace_size() bytes (16-byte aligned). For M <= 8 that is every shape with at least
 * 8 blocks of K. For M > 8 it is the shapes whose unsplit grid is small (fewer than 128 tiles of 32
 * rows by 128 columns and K >= 512: K is split), and the shapes that run more than 256 tiles of 64
 * rows by 128 columns but fill less than 90% of their rounds of 256 workgroups (such as M=256,
 * N=12288: the tiles' 32-row blocks are dealt out in equal runs to 256 workgroups, and the runs
 * that share a tile add their partials). mxmatvec_workspace_size returns 0 for the other shapes,
 * which never touch the buffer.
 *  - The buffer must be zero-filled once before its first use (hipMemset, or any zeroed
 *    allocation). Every call leaves its counters at zero again, so the buffer stays valid for any
 *    later call whose requirement it meets.
 *  - The library cannot check the contents. A buffer whose counter region is not zero, or one that
 *    two calls use at the same time (calls on different streams, or a graph replay that overlaps an
 *    eager call), makes the wrong workgroup of a column strip (or none) add the partial sums: that
 *    strip of y is then wrong or left unwritten, and later calls on the same buffer inherit the
 *    stale counter. Zero the counter region again to recover. Calls that may overlap in time need
 *    separate workspaces.
 *  - The last workgroup of each strip (or tile) adds the partial sums in a fixed order, so results
 *    are deterministic.
 *  - With workspace == NULL, or workspace_bytes below the requirement, K is not split across
 *    workgroups and the buffer is not touched (same results up to fp32 summation order; slower
 *    when N is small compared with the number of compute units).
 */
int mxmatvec_run(int M, int N, int K, const void* x, const void* W, int fw, const void* Ws, void* y,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes mxmatvec_run uses for this shape (0: none needed, or an invalid shape). For
 * 1 <= M <= 8 the requirement never decreases as M grows for fixed N, K and fw; for M > 8 it can
 * (a larger M has more tiles and so fewer K splits). */
size_t mxmatvec_workspace_size(int M, int N, int K, int fw);

/* Size of the library's static scratch array (17 MiB), the most workspace mxmatvec_run_noalloc can
 * use. Every valid shape fits: the requirement is 16 KiB of counters, then fp32 partials of at most
 * 16 MiB (M <= 8: at most 16 splits x 8 rows x 128 strips of 256 columns; M > 8: at most 256 splits
 * x tiles of 32 x 128, 4 MiB, or two 64 x 128 tiles for each of at most 256 workgroups, 16 MiB). */
#define MXMATVEC_SCRATCH_BYTES ((size_t)17 << 20)

/*
 * mxmatvec_run_noalloc -- mxmatvec_run for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same operation, arguments,
 * shape rules and kernels as mxmatvec_run with a large enough workspace, and the same results bit
 * for bit, but the split kernel's workspace is a static device array inside the library
 * (MXMATVEC_SCRATCH_BYTES per GPU, held until the process ends). Nothing is allocated, by the
 * library or any library it calls.
 *  - A shape whose workspace requirement (mxmatvec_workspace_size) exceeded MXMATVEC_SCRATCH_BYTES
 *    would return MX_ERR_SCRATCH before anything is queued; no valid shape does (see above).
 *  - All calls on one GPU share that GPU's array, which keeps the last call's contents (its
 *    counters are back at zero after every call). Calls that overlap in time on one GPU (different
 *    streams, or a captured graph replaying beside another call) race on it and give wrong results:
 *    serialise them, or use mxmatvec_run with separate workspaces.
 *  - The first call on a GPU looks up the array's device address and queues a small kernel that
 *    zeroes the counters on `stream` ahead of its own work.
 */
int mxmatvec_run_noalloc(int M, int N, int K, const void* x, const void* W, int fw, const void* Ws, void* y,
                         void* stream);

/* ------------------------------------------------------------------------------------------ */
/* Codecs on the GPU (bit-exact with the host codecs below).                                    */
/* ------------------------------------------------------------------------------------------ */

/*
 * mx_pack_run -- quantise fp32 src [rows][cols] on the GPU. The pages start from tensors already
 * held in a quantized data type with an E8M0 scale plane (WWDC26 session 330 summary, the
 * multi-plane tensor of data and scale factors, blockFactors {32,1}); the scale rules below are the
 * synthetic workloads' ("floor(log2(absmax)) - emax + 127" per 32-element block along K; symmetric
 * int8 with scale = absmax/127 per 32-row group, and an int4 variant of it).
 *  f = MX_E4M3 / MX_E5M2 / MX_E2M3 / MX_E3M2 / MX_E2M1: blocks of 32 along cols. Per block:
 *      amax = max|x|; E = clamp(floor(log2 amax) - emax + 127, 0, 254) with emax = 8 (E4M3),
 *      15 (E5M2), 2 (E2M3), 4 (E3M2) or 2 (E2M1), the exponent of the format's largest element
 *      (amax = 0 gives E = 0); codes = x * 2^(127-E) rounded to the nearest element value, ties to
 *      the even code, saturated to +-448 / +-57344 / +-7.5 / +-28 / +-6, sign kept (negative
 *      values that round to zero give -0). A block holding Inf or NaN gets E = 0xFF and zero
 *      codes. codes: [rows][cols] (E4M3, E5M2), [rows][3*cols/4] (E2M3, E3M2: element j in bits
 *      6j..6j+5 of the row as a little-endian bit stream) or [rows][cols/2] (E2M1); scales: E8M0
 *      [rows][cols/32]. cols % 32 == 0.
 *  f = MX_INT8 / MX_INT4: src is a weight W [K=rows][N=cols], blocks of 32 along rows. Per
 *      column and block: s = fp16(amax / qmax) (fp32 division, nearest-even to fp16) with
 *      qmax = 127 or 7; q = clamp(round_half_even(fp32(w / s)), -qmax, qmax), q = 0 where
 *      s = 0. A block holding Inf or NaN gets s = NaN (0x7E00) and q = 0. codes: int8
 *      [rows][cols] or packed int4 [rows][cols/2] (TensorOps notes, "VALIDATED ON M4 MAX",
 *      fact 5); scales: binary16 [rows/32][cols]. rows % 32 == 0; cols % 2 == 0 for MX_INT4.
 * Errors: MX_ERR_NULL, MX_ERR_SHAPE, MX_ERR_FORMAT (f not listed), MX_ERR_ALIGN, MX_ERR_ARCH,
 * MX_ERR_LAUNCH; nothing is queued on an error.
 */
int mx_pack_run(int f, const float* src, int rows, int cols, void* codes, void* scales, void* stream);

/*
 * mx_unpack_run -- dequantise to fp32 on the GPU: out = fp32(value * scale), the exact product
 * rounded once to fp32 (nearest even; subnormals kept; overflow gives +-Inf; NaN propagates). This
 * is the dequantisation the pages' matmul applies to each element in the kernel (TensorOps notes,
 * "Scale planes": value times its block's power-of-two scale; "Kernel-phase findings": int weights
 * times their fp16 block scale), written out as its own result. Layouts as in mx_pack_run (MX:
 * scales along cols; INT8/INT4: scales along rows). Errors as for mx_pack_run.
 */
int mx_unpack_run(int f, const void* codes, const void* scales, int rows, int cols, float* out,
                  void* stream);

/* ------------------------------------------------------------------------------------------ */
/* Host codecs (CPU, synchronous, same definitions and layouts as the GPU codecs).              */
/* ------------------------------------------------------------------------------------------ */

int mx_pack_host(int f, const float* src, int64_t rows, int64_t cols, void* codes, void* scales);
int mx_unpack_host(int f, const void* codes, const void* scales, int64_t rows, int64_t cols, float* out);

/* Single-element encoder/decoder of the host codec. mx_encode_host: f = MX_E4M3, MX_E5M2,
 * MX_E2M3, MX_E3M2 or MX_E2M1, nearest code, ties to even, saturating, sign kept (0 for other f).
 * mx_decode_host: f = MX_E4M3, MX_E5M2, MX_E2M3 / MX_E3M2 (low 6 bits), MX_E2M1 (low nibble),
 * MX_E8M0, MX_INT8 or MX_INT4 (low nibble); NaN for other f. */
uint8_t mx_encode_host(int f, float v);
float mx_decode_host(int f, uint8_t code);

#ifdef __cplusplus
}
#endif
#endif /* MXGEMM_H */
