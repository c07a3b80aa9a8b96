"""GPU GEMMs (MXFP8, MXFP4, fp16) against the oracle.

Inputs are seeded fp32 sources; the GPU quantises them with mx_pack_run, the oracle with its own
quantiser, and the two code/scale planes must agree bit for bit before the products are compared.
Products must meet |C_gpu - C_ref| <= 2^-10 |C_ref| + 1e-3 sqrt(K) R (R = rms of |a_mk b_kn|), with
NaN positions equal. Small and ragged shapes are compared on every output; the full-size
workloads on sampled outputs (all four corners included) plus a finiteness check of all of C, which
starts NaN-filled, so that check also proves every output was written.
"""
import os

import numpy as np
import pytest
import torch

from block_scaled_quantized_amd import synth
from gpu_common import dev, empty, gpu_gemm, gpu_mx_pack, host, nan_f16, require_gpu, say

pytestmark = pytest.mark.gpu


def R_of(orc, fmt, A, SA, B, SB, M, N, K):
    return orc.rms_ab(orc.dequant(fmt, A, SA, M, K), orc.dequant(fmt, B, SB, N, K).T)


def mx_case(orc, api, fmt, M, N, K, seed, sigma_b=1.0, tile=None):
    a_src = synth.normal((M, K), 1.0, seed)
    b_src = synth.normal((N, K), sigma_b, seed + 1)   # B drawn in its K-contiguous storage order
    A, SA = gpu_mx_pack(api, fmt, a_src)
    B, SB = gpu_mx_pack(api, fmt, b_src)
    oA, oSA = orc.mx_quantize(fmt, a_src)
    oB, oSB = orc.mx_quantize(fmt, b_src)
    assert np.array_equal(host(A), oA) and np.array_equal(host(SA), oSA)
    assert np.array_equal(host(B), oB) and np.array_equal(host(SB), oSB)
    old = os.environ.get("MXGEMM_TILE")
    if tile is not None:
        os.environ["MXGEMM_TILE"] = str(tile)
    try:
        C = gpu_gemm(api, fmt, A, SA, B, SB, M, N, K)
    finally:
        if tile is not None:
            if old is None:
                del os.environ["MXGEMM_TILE"]
            else:
                os.environ["MXGEMM_TILE"] = old
    return C, (oA, oSA, oB, oSB)


@pytest.mark.parametrize("fmt", [0, 4])
def test_mx_small_config_full(orc, fmt):
    """MXFP8 M=128, N=256, K=128 (and the same shape in MXFP4): every output."""
    api = require_gpu()
    M, N, K = 128, 256, 128
    say(f"mx small fmt={fmt}")
    C, (oA, oSA, oB, oSB) = mx_case(orc, api, fmt, M, N, K, synth.seed_for(synth.MXFP8_SMALL, 0))
    ref = orc.mxgemm(fmt, fmt, oA, oSA, oB, oSB, M, N, K)
    ok, ratio, bad = orc.check(C, ref, K, R_of(orc, fmt, oA, oSA, oB, oSB, M, N, K))
    assert ok, (ratio, bad)


@pytest.mark.parametrize("fmt", [0, 4])
@pytest.mark.parametrize("tile", [0, 1, 2, 3, 4, 5, 6, 7, 8, 9])
def test_mx_every_tile_ragged(orc, fmt, tile):
    """Each tile configuration on a shape spanning several tiles with ragged M, N and K tails."""
    api = require_gpu()
    M, N, K = 300, 520, 416          # K = 13 blocks: partial last stage for both formats
    say(f"mx ragged fmt={fmt} tile={tile}")
    C, (oA, oSA, oB, oSB) = mx_case(orc, api, fmt, M, N, K, 4242 + tile, tile=tile)
    ref = orc.mxgemm(fmt, fmt, oA, oSA, oB, oSB, M, N, K)
    ok, ratio, bad = orc.check(C, ref, K, R_of(orc, fmt, oA, oSA, oB, oSB, M, N, K))
    assert ok, (ratio, bad)


@pytest.mark.parametrize("fmt", [0, 4])
@pytest.mark.parametrize("tile", [6, 7])
@pytest.mark.parametrize("K", [128, 256, 512, 1024])
def test_mx_pingpong_ragged_mn(orc, fmt, tile, K):
    """The 8-wave ping-pong kernels (whole stages only: K % 128 (E4M3) / 256 (E2M1) == 0) on ragged
    M and N, from one and two stages up to several."""
    api = require_gpu()
    if fmt == 4 and K % 256:
        pytest.skip("E2M1 stages are 256 wide")
    M, N = 300, 520
    say(f"mx ping-pong fmt={fmt} tile={tile} K={K}")
    C, (oA, oSA, oB, oSB) = mx_case(orc, api, fmt, M, N, K, 999 + K + tile, tile=tile)
    ref = orc.mxgemm(fmt, fmt, oA, oSA, oB, oSB, M, N, K)
    ok, ratio, bad = orc.check(C, ref, K, R_of(orc, fmt, oA, oSA, oB, oSB, M, N, K))
    assert ok, (ratio, bad)


@pytest.mark.parametrize("fmt,M,N,K", [
    (0, 300, 520, 512), (0, 300, 520, 1024), (0, 257, 260, 4096), (0, 1, 4, 512), (0, 512, 512, 1536),
    (0, 33, 1028, 2560),
    (4, 300, 520, 1024), (4, 257, 260, 4096), (4, 1, 4, 1024), (4, 512, 512, 2048), (4, 33, 1028, 3072),
])
@pytest.mark.parametrize("tile", [8, 9, 10])
def test_mx_ring_ragged(orc, fmt, M, N, K, tile):
    """The 4-stage ring kernels, 256x256 (tile 8), 256x224 (tile 9) and 256x192 (tile 10) tiles
    (N % 4 == 0; K % 512 == 0 for E4M3, K % 1024 == 0 for E2M1): one scale group up to several,
    partial tiles in M and N, a single row and column strip."""
    api = require_gpu()
    say(f"mx ring tile={tile} fmt={fmt} M={M} N={N} K={K}")
    C, (oA, oSA, oB, oSB) = mx_case(orc, api, fmt, M, N, K, 31 + M + N + K, tile=tile)
    ref = orc.mxgemm(fmt, fmt, oA, oSA, oB, oSB, M, N, K)
    ok, ratio, bad = orc.check(C, ref, K, R_of(orc, fmt, oA, oSA, oB, oSB, M, N, K))
    assert ok, (ratio, bad)


@pytest.mark.parametrize("fmt", [0, 4])
@pytest.mark.parametrize("shape", [(1, 1, 32), (1, 8, 64), (17, 3, 96), (5, 129, 4096), (64, 64, 288)])
def test_mx_degenerate_shapes(orc, fmt, shape):
    api = require_gpu()
    M, N, K = shape
    say(f"mx degenerate fmt={fmt} shape={shape}")
    C, (oA, oSA, oB, oSB) = mx_case(orc, api, fmt, M, N, K, 77 + M + N + K)
    ref = orc.mxgemm(fmt, fmt, oA, oSA, oB, oSB, M, N, K)
    ok, ratio, bad = orc.check(C, ref, K, R_of(orc, fmt, oA, oSA, oB, oSB, M, N, K))
    assert ok, (ratio, bad)


def small_codes(fmt, shape, seed):
    """Random codes of magnitude <= 4 (E4M3: exponent field <= 8, every subnormal) or any E2M1
    byte, so that sums of a few hundred products stay inside the fp16 range."""
    if fmt == 4:
        return synth.random_bytes(shape, seed)
    b = synth.random_bytes(shape, seed)                  # sign and mantissa bits
    e = synth.random_ints(shape, 0, 8, seed + 1000)      # exponent field 0..8: |value| < 2
    return ((b & 0x87) | (e << 3)).astype(np.uint8)


def test_mx_fp16_overflow_is_inf(orc):
    """Sums beyond 65504 are written as +-Inf (fp16 nearest-even overflow) with the right sign."""
    api = require_gpu()
    M, N, K = 32, 32, 256
    say("mx fp16 overflow")
    A = synth.random_bytes((M, K), 25, exclude=(0x7F, 0xFF))
    B = np.full((N, K), 0x7E, np.uint8)                   # 448 everywhere
    A[:, :] = 0x7E
    A[1::2, :] = 0xFE                                      # odd rows -448
    SA = np.full((M, K // 32), 127, np.uint8)
    SB = np.full((N, K // 32), 127, np.uint8)
    C = gpu_gemm(api, 0, dev(A), dev(SA), dev(B), dev(SB), M, N, K)
    assert np.all(C[0::2] == np.inf) and np.all(C[1::2] == -np.inf)
    ref = orc.mxgemm(0, 0, A, SA, B, SB, M, N, K)
    ok, ratio, bad = orc.check(C, ref, K, R_of(orc, 0, A, SA, B, SB, M, N, K))
    assert ok, (ratio, bad)


@pytest.mark.parametrize("fmt", [0, 4])
def test_mx_nonfinite_and_extreme_scales(orc, fmt):
    """NaN scale (0xFF), NaN E4M3 codes, the smallest and largest scales."""
    api = require_gpu()
    M, N, K = 64, 96, 256
    say(f"mx nonfinite fmt={fmt}")
    rb = K if fmt == 0 else K // 2
    A = small_codes(fmt, (M, rb), 5)
    B = small_codes(fmt, (N, rb), 6)
    SA = synth.random_ints((M, K // 32), 118, 128, 7)
    SB = synth.random_ints((N, K // 32), 118, 128, 8)
    SA[3, 2] = 0xFF                      # NaN scale: row 3
    SB[10, 5] = 0xFF                     # NaN scale: column 10
    SA[5, 1:] = 0                        # 2^-127 in row 5 (tiny but finite products)
    SA[:, 0] = 1                         # block 0: 2^-126 on every row of A ...
    SB[20, 0] = 254                      # ... so the largest scale 2^127 on column 20 stays in range
    if fmt == 0:
        A[7, 33] = 0x7F                  # NaN code: row 7
        B[30, 200] = 0xFF                # NaN code: column 30
    C = gpu_gemm(api, fmt, dev(A), dev(SA), dev(B), dev(SB), M, N, K)
    ref = orc.mxgemm(fmt, fmt, A, SA, B, SB, M, N, K)
    fin = ~np.isnan(ref)
    R = orc.rms_ab(np.nan_to_num(orc.dequant(fmt, A, SA, M, K)), np.nan_to_num(orc.dequant(fmt, B, SB, N, K)).T)
    assert np.array_equal(np.isnan(C), ~fin)
    ok, ratio, bad = orc.check(C[fin], ref[fin], K, R)
    assert ok, (ratio, bad)


@pytest.mark.parametrize("fmt,tile,M,N,K", [
    (0, 8, 300, 520, 1024), (4, 8, 300, 520, 1024), (0, 7, 300, 520, 512), (4, 4, 300, 520, 416),
    (0, 3, 17, 40, 96), (0, 9, 257, 260, 512),
])
def test_mx_relu_epilogue(orc, fmt, tile, M, N, K):
    """MXGEMM_RELU: C = max(A*B, 0) for every kernel family (ring, ping-pong, 8-wave, 4-wave)."""
    api = require_gpu()
    say(f"mx relu fmt={fmt} tile={tile} M={M} N={N} K={K}")
    a_src = synth.normal((M, K), 1.0, 600 + tile)
    b_src = synth.normal((N, K), 1.0, 601 + tile)
    A, SA = gpu_mx_pack(api, fmt, a_src)
    B, SB = gpu_mx_pack(api, fmt, b_src)
    oA, oSA = orc.mx_quantize(fmt, a_src)
    oB, oSB = orc.mx_quantize(fmt, b_src)
    old = os.environ.get("MXGEMM_TILE")
    os.environ["MXGEMM_TILE"] = str(tile)
    try:
        C = gpu_gemm(api, fmt, A, SA, B, SB, M, N, K, flags=api.MXGEMM_RELU)
    finally:
        if old is None:
            del os.environ["MXGEMM_TILE"]
        else:
            os.environ["MXGEMM_TILE"] = old
    ref = orc.relu(orc.mxgemm(fmt, fmt, oA, oSA, oB, oSB, M, N, K))
    assert (C >= 0).all() and (C == 0).mean() > 0.3      # about half the outputs are clipped
    ok, ratio, bad = orc.check(C, ref, K, R_of(orc, fmt, oA, oSA, oB, oSB, M, N, K))
    assert ok, (ratio, bad)


def test_relu_epilogue_nan_and_f16(orc):
    """ReLU maps a NaN product (NaN scale) to 0, and applies to the fp16 GEMM too."""
    api = require_gpu()
    M, N, K = 64, 96, 256
    say("relu nan / f16")
    A = small_codes(0, (M, K), 5)
    B = small_codes(0, (N, K), 6)
    SA = synth.random_ints((M, K // 32), 118, 128, 7)
    SB = synth.random_ints((N, K // 32), 118, 128, 8)
    SA[3, 2] = 0xFF
    C = gpu_gemm(api, 0, dev(A), dev(SA), dev(B), dev(SB), M, N, K, flags=api.MXGEMM_RELU)
    ref = orc.mxgemm(0, 0, A, SA, B, SB, M, N, K)
    assert np.isnan(ref[3]).all() and (C[3] == 0).all()
    R = orc.rms_ab(np.nan_to_num(orc.dequant(0, A, SA, M, K)), orc.dequant(0, B, SB, N, K).T)
    ok, ratio, bad = orc.check(C, orc.relu(ref), K, R)
    assert ok, (ratio, bad)
    A16 = synth.uniform_pm1((M, K), 70).astype(np.float16)
    B16 = synth.uniform_pm1((K, N), 71).astype(np.float16)
    C16 = gpu_gemm(api, api.MX_F16, dev(A16), None, dev(B16), None, M, N, K, flags=api.MXGEMM_RELU)
    ok, ratio, bad = orc.check(C16, orc.relu(orc.gemm_f16(A16, B16)), K,
                               orc.rms_ab(A16.astype(np.float64), B16.astype(np.float64)))
    assert ok, (ratio, bad)


@pytest.mark.parametrize("fa,fb", [(0, 4), (4, 0)])
@pytest.mark.parametrize("tile,M,N,K", [
    (8, 300, 520, 1024), (8, 257, 260, 4096), (8, 1, 4, 512), (8, 33, 1028, 2560), (9, 300, 520, 512),
    (9, 257, 260, 1536),
])
def test_mx_mixed_pairs(orc, fa, fb, tile, M, N, K):
    """Mixed MX pairs (E4M3 A x E2M1 B and E2M1 A x E4M3 B) on the ring kernels, every output."""
    api = require_gpu()
    say(f"mx mixed fa={fa} fb={fb} tile={tile} M={M} N={N} K={K}")
    a_src = synth.normal((M, K), 1.0, 700 + M + K)
    b_src = synth.normal((N, K), 1.0, 701 + N + K)
    A, SA = gpu_mx_pack(api, fa, a_src)
    B, SB = gpu_mx_pack(api, fb, b_src)
    oA, oSA = orc.mx_quantize(fa, a_src)
    oB, oSB = orc.mx_quantize(fb, b_src)
    assert np.array_equal(host(A), oA) and np.array_equal(host(B), oB)
    old = os.environ.get("MXGEMM_TILE")
    os.environ["MXGEMM_TILE"] = str(tile)
    try:
        C = gpu_gemm(api, fa, A, SA, B, SB, M, N, K, fb=fb)
    finally:
        if old is None:
            del os.environ["MXGEMM_TILE"]
        else:
            os.environ["MXGEMM_TILE"] = old
    ref = orc.mxgemm(fa, fb, oA, oSA, oB, oSB, M, N, K)
    R = orc.rms_ab(orc.dequant(fa, oA, oSA, M, K), orc.dequant(fb, oB, oSB, N, K).T)
    ok, ratio, bad = orc.check(C, ref, K, R)
    assert ok, (ratio, bad)


@pytest.mark.parametrize("fa,fb", [(1, 1), (0, 1), (1, 0), (1, 4), (4, 1)])
@pytest.mark.parametrize("M,N,K", [(300, 520, 512), (257, 260, 1536), (64, 1028, 1024)])
def test_mx_e5m2_pairs(orc, fa, fb, M, N, K):
    """Pairs with an E5M2 operand on the ring (the MFMA's bf8 format code), every output: the GPU's
    E5M2 pack must equal the oracle's, and the product must meet the bound."""
    api = require_gpu()
    say(f"mx e5m2 fa={fa} fb={fb} M={M} N={N} K={K}")
    a_src = synth.normal((M, K), 1.0, 800 + M + K)
    b_src = synth.normal((N, K), 0.02, 801 + N + K)
    A, SA = gpu_mx_pack(api, fa, a_src)
    B, SB = gpu_mx_pack(api, fb, b_src)
    oA, oSA = orc.mx_quantize(fa, a_src)
    oB, oSB = orc.mx_quantize(fb, b_src)
    assert np.array_equal(host(A), oA) and np.array_equal(host(SA), oSA)
    assert np.array_equal(host(B), oB) and np.array_equal(host(SB), oSB)
    C = gpu_gemm(api, fa, A, SA, B, SB, M, N, K, fb=fb)
    ref = orc.mxgemm(fa, fb, oA, oSA, oB, oSB, M, N, K)
    R = orc.rms_ab(orc.dequant(fa, oA, oSA, M, K), orc.dequant(fb, oB, oSB, N, K).T)
    ok, ratio, bad = orc.check(C, ref, K, R)
    assert ok, (ratio, bad)


@pytest.mark.parametrize("fa,fb", [(2, 2), (3, 3), (2, 3), (3, 2)])
@pytest.mark.parametrize("M,N,K", [(300, 520, 512), (257, 260, 1536), (64, 1028, 1024)])
def test_mx_fp6_pairs(orc, fa, fb, M, N, K):
    """FP6 pairs (E2M3 / E3M2, 48-byte stage rows) on the ring, every output: the GPU's FP6 pack must
    equal the oracle's, and the product must meet the bound."""
    api = require_gpu()
    say(f"mx fp6 fa={fa} fb={fb} M={M} N={N} K={K}")
    a_src = synth.normal((M, K), 1.0, 900 + M + K)
    b_src = synth.normal((N, K), 0.02, 901 + N + K)
    A, SA = gpu_mx_pack(api, fa, a_src)
    B, SB = gpu_mx_pack(api, fb, b_src)
    oA, oSA = orc.mx_quantize(fa, a_src)
    oB, oSB = orc.mx_quantize(fb, b_src)
    assert np.array_equal(host(A), oA) and np.array_equal(host(SA), oSA)
    assert np.array_equal(host(B), oB) and np.array_equal(host(SB), oSB)
    C = gpu_gemm(api, fa, A, SA, B, SB, M, N, K, fb=fb)
    ref = orc.mxgemm(fa, fb, oA, oSA, oB, oSB, M, N, K)
    R = orc.rms_ab(orc.dequant(fa, oA, oSA, M, K), orc.dequant(fb, oB, oSB, N, K).T)
    ok, ratio, bad = orc.check(C, ref, K, R)
    assert ok, (ratio, bad)


def test_mx_fp6_unit_scales_exact(orc):
    """E2M3 x E3M2 at unit scales: every product is a multiple of 2^-7 of magnitude at most 210, so
    with K=512 every partial sum is below 2^17 and exact in fp32: the GPU must equal the oracle
    after the fp16 rounding."""
    api = require_gpu()
    M, N, K = 256, 512, 512
    say("mx fp6 unit scales exact")
    g = np.random.Generator(np.random.PCG64(911))

    def pack(codes):
        bits = ((codes[..., None] >> np.arange(6)) & 1).astype(np.uint8).reshape(codes.shape[0], -1)
        return np.ascontiguousarray(np.packbits(bits, axis=1, bitorder="little"))
    ca, cb = g.integers(0, 64, (M, K)), g.integers(0, 64, (N, K))
    SA = np.full((M, K // 32), 127, np.uint8)
    SB = np.full((N, K // 32), 127, np.uint8)
    A, B = pack(ca), pack(cb)
    C = gpu_gemm(api, 2, dev(A), dev(SA), dev(B), dev(SB), M, N, K, fb=3)
    ref = orc.mxgemm(2, 3, A, SA, B, SB, M, N, K)
    assert np.abs(ref).max() < 60000
    assert np.array_equal(C, ref.astype(np.float16).astype(np.float64))


def test_mx_e5m2_unit_scales_exact(orc):
    """E5M2 x E5M2 at unit scales on codes whose products and sums are exact in fp32: the GPU must
    equal the oracle (its plain fp8 matmul) after the fp16 rounding, output for output."""
    api = require_gpu()
    M, N, K = 256, 512, 1024
    say("mx e5m2 unit scales exact")
    g = np.random.Generator(np.random.PCG64(811))

    def codes(shape):   # exponent fields 13..17: values 2^-2 .. 1.75*2^2, signs random
        return ((g.integers(0, 2, size=shape) << 7) | (g.integers(13, 18, size=shape) << 2)
                | g.integers(0, 4, size=shape)).astype(np.uint8)
    A, B = codes((M, K)), codes((N, K))
    SA = np.full((M, K // 32), 127, np.uint8)
    SB = np.full((N, K // 32), 127, np.uint8)
    C = gpu_gemm(api, 1, dev(A), dev(SA), dev(B), dev(SB), M, N, K)
    ref = orc.mxgemm(1, 1, A, SA, B, SB, M, N, K)
    assert np.abs(ref).max() < 60000
    assert np.array_equal(C, ref.astype(np.float16).astype(np.float64))


def test_mx_unit_scales_fp8_exact_products(orc):
    """Scale 127 everywhere: the oracle equals a plain fp8 matmul; the GPU must match within the bound."""
    api = require_gpu()
    M, N, K = 256, 256, 512
    say("mx unit scales")
    A = small_codes(0, (M, K), 15)
    B = small_codes(0, (N, K), 16)
    SA = np.full((M, K // 32), 127, np.uint8)
    SB = np.full((N, K // 32), 127, np.uint8)
    C = gpu_gemm(api, 0, dev(A), dev(SA), dev(B), dev(SB), M, N, K)
    ref = orc.mxgemm(0, 0, A, SA, B, SB, M, N, K)
    ok, ratio, bad = orc.check(C, ref, K, R_of(orc, 0, A, SA, B, SB, M, N, K))
    assert ok, (ratio, bad)


@pytest.mark.parametrize("name,fmt,M,N,K,sigma_b,wl", [
    ("mxfp8_prefill", 0, 2048, 14336, 4096, 0.02, synth.MXFP8_PREFILL),
    ("mxfp4_large", 4, 4096, 8192, 8192, 1.0, synth.MXFP4_LARGE),
])
def test_mx_full_size_sampled(orc, name, fmt, M, N, K, sigma_b, wl):
    api = require_gpu()
    say(f"full size {name}")
    a_src = synth.normal((M, K), 1.0, synth.seed_for(wl, 0))
    b_src = synth.normal((N, K), sigma_b, synth.seed_for(wl, 1))
    A, SA = gpu_mx_pack(api, fmt, a_src)
    B, SB = gpu_mx_pack(api, fmt, b_src)
    C = gpu_gemm(api, fmt, A, SA, B, SB, M, N, K)
    assert np.isfinite(C).all()
    oA, oSA = orc.mx_quantize(fmt, a_src)
    oB, oSB = orc.mx_quantize(fmt, b_src)
    del a_src, b_src
    assert np.array_equal(host(SA), oSA) and np.array_equal(host(SB), oSB)
    assert np.array_equal(host(A), oA) and np.array_equal(host(B), oB)
    ms, ns = synth.sample_points(M, N, 2048, 99)
    ref = orc.mxgemm_points(fmt, fmt, oA, oSA, oB, oSB, K, ms, ns)
    ok, ratio, bad = orc.check(C[ms, ns], ref, K, R_of(orc, fmt, oA, oSA, oB, oSB, M, N, K))
    say(f"{name}: worst err/bound {ratio:.3f}")
    assert ok, (ratio, bad)


def fp16_case(orc, api, M, N, K, seed, tile=None):
    A = synth.uniform_pm1((M, K), seed).astype(np.float16)
    B = synth.uniform_pm1((K, N), seed + 1).astype(np.float16)
    old = os.environ.get("MXGEMM_TILE")
    if tile is not None:
        os.environ["MXGEMM_TILE"] = str(tile)
    try:
        C = gpu_gemm(api, api.MX_F16, dev(A), None, dev(B), None, M, N, K)
    finally:
        if tile is not None:
            if old is None:
                del os.environ["MXGEMM_TILE"]
            else:
                os.environ["MXGEMM_TILE"] = old
    return A, B, C


@pytest.mark.parametrize("tile", [0, 1, 2, 3, 4, 5, 6, 7, 8, 9])
def test_f16_every_tile_ragged(orc, tile):
    api = require_gpu()
    M, N, K = 300, 520, 200
    say(f"f16 ragged tile={tile}")
    A, B, C = fp16_case(orc, api, M, N, K, 500 + tile, tile=tile)
    ref = orc.gemm_f16(A, B)
    ok, ratio, bad = orc.check(C, ref, K, orc.rms_ab(A.astype(np.float64), B.astype(np.float64)))
    assert ok, (ratio, bad)


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (300, 512, 512), (520, 768, 1280), (40, 256, 768)])
def test_f16_ring(orc, M, N, K):
    """The fp16 ring (tile 8 where N % 256 == 0 and K % 256 == 0): B staged as K-rows and read
    through transposing LDS loads; one group of 8 stages up to several, partial tiles in M."""
    api = require_gpu()
    say(f"f16 ring M={M} N={N} K={K}")
    A, B, C = fp16_case(orc, api, M, N, K, 700 + M + N + K, tile=8)
    ref = orc.gemm_f16(A, B)
    ok, ratio, bad = orc.check(C, ref, K, orc.rms_ab(A.astype(np.float64), B.astype(np.float64)))
    assert ok, (ratio, bad)


def test_f16_ring_exact_integers(orc):
    """Small integer operands make every product and partial sum exact in fp32, so the fp16 ring's
    output must equal the oracle's sum rounded to fp16 exactly: any A/B element paired with the
    wrong K shows up."""
    api = require_gpu()
    M, N, K = 512, 768, 768
    say("f16 ring exact integers")
    A = (synth.random_ints((M, K), 0, 6, 720).astype(np.int64) - 3).astype(np.float16)
    B = (synth.random_ints((K, N), 0, 6, 721).astype(np.int64) - 3).astype(np.float16)
    old = os.environ.get("MXGEMM_TILE")
    os.environ["MXGEMM_TILE"] = "8"
    try:
        C = gpu_gemm(api, api.MX_F16, dev(A), None, dev(B), None, M, N, K)
    finally:
        if old is None:
            del os.environ["MXGEMM_TILE"]
        else:
            os.environ["MXGEMM_TILE"] = old
    ref = orc.gemm_f16(A, B)
    assert np.abs(ref).max() < 2048                 # integers, exact in fp16
    assert np.array_equal(C.astype(np.float64), ref)


@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (300, 520, 1024), (512, 1024, 512), (40, 2056, 1536),
                                   (1024, 2048, 2048), (1, 8, 512), (257, 264, 512), (64, 1000, 1024),
                                   (33, 8, 2560)])
def test_f16_pp_ring(orc, M, N, K):
    """fp16 on the ping-pong ring (tile 11 where K % 512 == 0 and N % 8 == 0): A in E4M3's byte
    layout, B staged per slot as 64 K-rows of 512 bytes and read through transposing LDS loads. One
    tile up to 32 (8 and more: the XCD remap), ragged M down to a single row, ragged N down to 8
    columns (N % 256 != 0: the last tile's extra columns read later K rows, or zeros past the end
    of B, and are never stored), 4 to 20 groups of K; every output against the oracle."""
    api = require_gpu()
    plan = with_tile(11, lambda: api.mxgemm_create(M, N, K, api.MX_F16, api.MX_F16))
    assert list(api.mxgemm_plan_info(plan)) == [256, 256, 32, 4]
    plan.close()
    say(f"f16 pp ring M={M} N={N} K={K}")
    A, B, C = fp16_case(orc, api, M, N, K, 900 + M + N + K, tile=11)
    ref = orc.gemm_f16(A, B)
    ok, ratio, bad = orc.check(C, ref, K, orc.rms_ab(A.astype(np.float64), B.astype(np.float64)))
    assert ok, (ratio, bad)


def test_f16_pp_ring_exact_integers_and_relu(orc):
    """Small integer operands make every product and partial sum exact in fp32, so the fp16
    ping-pong ring's output must equal the oracle's sum rounded to fp16 exactly (any A or B element
    paired with the wrong K shows up); then the same with the ReLU epilogue."""
    api = require_gpu()
    M, N, K = 512, 776, 1024
    say("f16 pp ring exact integers, relu")
    A = (synth.random_ints((M, K), 0, 6, 920).astype(np.int64) - 3).astype(np.float16)
    B = (synth.random_ints((K, N), 0, 6, 921).astype(np.int64) - 3).astype(np.float16)
    ref = orc.gemm_f16(A, B)
    assert np.abs(ref).max() < 2048                 # integers, exact in fp16
    C = with_tile(11, lambda: gpu_gemm(api, api.MX_F16, dev(A), None, dev(B), None, M, N, K))
    assert np.array_equal(C, ref)
    Cr = with_tile(11, lambda: gpu_gemm(api, api.MX_F16, dev(A), None, dev(B), None, M, N, K, flags=api.MXGEMM_RELU))
    assert np.array_equal(Cr, np.maximum(ref, 0.0))


def test_f16_square_full_size_sampled(orc):
    """fp16 GEMM M=N=K=4096, U(-1,1) inputs, on the plan's own choice (the ping-pong ring)."""
    api = require_gpu()
    plan = api.mxgemm_create(4096, 4096, 4096, api.MX_F16, api.MX_F16)
    assert list(api.mxgemm_plan_info(plan)) == [256, 256, 32, 4]
    plan.close()
    M = N = K = 4096
    say("f16 square 4096")
    A, B, C = fp16_case(orc, api, M, N, K, synth.seed_for(synth.F16_SQUARE, 0))
    assert np.isfinite(C).all()
    ms, ns = synth.sample_points(M, N, 2048, 98)
    ref = orc.gemm_f16_points(A, B, ms, ns)
    ok, ratio, bad = orc.check(C[ms, ns], ref, K, orc.rms_ab(A.astype(np.float64), B.astype(np.float64)))
    say(f"f16 square: worst err/bound {ratio:.3f}")
    assert ok, (ratio, bad)


def with_tile(tile, fn):
    old = os.environ.get("MXGEMM_TILE")
    if tile is not None:
        os.environ["MXGEMM_TILE"] = str(tile)
    try:
        return fn()
    finally:
        if tile is not None:
            if old is None:
                del os.environ["MXGEMM_TILE"]
            else:
                os.environ["MXGEMM_TILE"] = old


def pair_case(orc, api, fa, fb, M, N, K, seed, tile=None, sigma_b=1.0):
    """GPU-packed MX operands of formats fa / fb, checked bit-exact against the oracle's packing;
    returns (C, oracle C, R)."""
    a_src = synth.normal((M, K), 1.0, seed)
    b_src = synth.normal((N, K), sigma_b, seed + 1)
    A, SA = gpu_mx_pack(api, fa, a_src)
    B, SB = gpu_mx_pack(api, fb, b_src)
    oA, oSA = orc.mx_quantize(fa, a_src)
    oB, oSB = orc.mx_quantize(fb, b_src)
    assert np.array_equal(host(A), oA) and np.array_equal(host(SA), oSA)
    assert np.array_equal(host(B), oB) and np.array_equal(host(SB), oSB)
    C = with_tile(tile, lambda: gpu_gemm(api, fa, A, SA, B, SB, M, N, K, fb=fb))
    ref = orc.mxgemm(fa, fb, oA, oSA, oB, oSB, M, N, K)
    R = orc.rms_ab(orc.dequant(fa, oA, oSA, M, K), orc.dequant(fb, oB, oSB, N, K).T)
    return C, ref, R


@pytest.mark.parametrize("fa,fb,tile,M,N,K", [
    (0, 0, 8, 512, 1024, 1024), (4, 4, 8, 512, 1024, 2048), (0, 4, 8, 512, 1024, 1024),
    (4, 0, 8, 512, 1024, 1024), (1, 1, 8, 512, 1024, 1024), (2, 3, 8, 512, 1024, 1024),
    (0, 0, 8, 1024, 1024, 512), (0, 0, 9, 512, 896, 1024), (4, 4, 9, 512, 896, 2048),
    (0, 4, 9, 512, 896, 1024), (0, 0, 10, 512, 768, 1024), (4, 4, 10, 512, 768, 2048),
])
def test_mx_ring_xcd_remap_every_output(orc, fa, fb, tile, M, N, K):
    """Ring grids of 8 or 16 tiles, where workgroup ids are remapped so that each XCD takes a
    contiguous range of tiles: every output against the oracle (the remap is a permutation of the
    tiles; a wrong one leaves tiles unwritten, and the NaN-filled C shows them)."""
    api = require_gpu()
    say(f"ring remap fa={fa} fb={fb} tile={tile} M={M} N={N} K={K}")
    C, ref, R = pair_case(orc, api, fa, fb, M, N, K, 1300 + M + N + K + tile, tile=tile)
    assert not np.isnan(C).any()
    ok, ratio, bad = orc.check(C, ref, K, R)
    assert ok, (ratio, bad)


def test_f16_ring_xcd_remap_every_output(orc):
    """The fp16 ring on a grid of 8 tiles (remapped), every output."""
    api = require_gpu()
    M, N, K = 512, 1024, 512
    say("f16 ring remap")
    A, B, C = fp16_case(orc, api, M, N, K, 1400, tile=8)
    assert not np.isnan(C).any()
    ok, ratio, bad = orc.check(C, orc.gemm_f16(A, B), K, orc.rms_ab(A.astype(np.float64), B.astype(np.float64)))
    assert ok, (ratio, bad)


def nonfinite_operands(fa, fb, M, N, K, seed):
    """Random codes of small magnitude with NaN scales, NaN codes (where the format has them) and
    the extreme scales 0x00 / 0xFE planted in rows of A and columns of B."""
    def codes(fmt, rows, s):
        if fmt == 4:
            return synth.random_bytes((rows, K // 2), s)
        if fmt in (2, 3):
            return synth.random_bytes((rows, K // 4 * 3), s)
        b = synth.random_bytes((rows, K), s)
        e = synth.random_ints((rows, K), 0, 8, s + 1000) if fmt == 0 else synth.random_ints((rows, K), 8, 16, s + 1000)
        return ((b & 0x87) | (e << 3)).astype(np.uint8) if fmt == 0 else ((b & 0x83) | (e << 2)).astype(np.uint8)
    A, B = codes(fa, M, seed), codes(fb, N, seed + 1)
    SA = synth.random_ints((M, K // 32), 118, 128, seed + 2)
    SB = synth.random_ints((N, K // 32), 118, 128, seed + 3)
    SA[3, 2] = 0xFF                      # NaN scale: row 3
    SB[10, K // 32 - 1] = 0xFF           # NaN scale in the last K-block: column 10
    SA[5, 1:] = 0                        # 2^-127: tiny but finite products in row 5
    SA[:, 0] = 1                         # block 0: 2^-126 on every row of A ...
    SB[20, 0] = 254                      # ... so the largest scale 2^127 on column 20 stays in range
    SB[N - 1, 3] = 0xFF                  # NaN scale on the last column (a partial tile's edge)
    if fa in (0, 1):
        A[7, K // 2 + 1] = 0x7F          # NaN code (E4M3 S.1111.111, E5M2 S.11111.11): row 7
    if fb in (0, 1):
        B[30, 200] = 0xFF                # NaN code: column 30
    return A, SA, B, SB


@pytest.mark.parametrize("fa,fb,tile,M,N,K", [
    (0, 0, 8, 300, 520, 512), (0, 0, 9, 257, 452, 1024), (0, 0, 10, 300, 388, 512),
    (4, 4, 8, 300, 520, 1024), (4, 4, 9, 257, 452, 1024), (4, 4, 10, 300, 388, 2048),
    (0, 4, 8, 300, 520, 512), (4, 0, 9, 300, 520, 1024), (1, 1, 8, 300, 520, 512), (1, 4, 8, 64, 260, 1024),
    (2, 3, 8, 300, 520, 512),
])
def test_mx_ring_nonfinite_and_extreme_scales(orc, fa, fb, tile, M, N, K):
    """The ring kernels with NaN scales, NaN codes and the extreme scales: NaN positions equal the
    oracle's and every finite output meets the bound (each operand's scales reach the MFMA through
    their own op_sel byte packing, so a scale fed to the wrong K-step or row shows up)."""
    api = require_gpu()
    say(f"ring nonfinite fa={fa} fb={fb} tile={tile} M={M} N={N} K={K}")
    A, SA, B, SB = nonfinite_operands(fa, fb, M, N, K, 2000 + tile + fa + fb)
    C = with_tile(tile, lambda: gpu_gemm(api, fa, dev(A), dev(SA), dev(B), dev(SB), M, N, K, fb=fb))
    ref = orc.mxgemm(fa, fb, A, SA, B, SB, M, N, K)
    assert np.isnan(ref[3]).all() and np.isnan(ref[:, 10]).all() and np.isnan(ref[:, N - 1]).all()
    R = orc.rms_ab(np.nan_to_num(orc.dequant(fa, A, SA, M, K)), np.nan_to_num(orc.dequant(fb, B, SB, N, K)).T)
    ok, ratio, bad = orc.check(C, ref, K, R)
    assert ok, (ratio, bad)


@pytest.mark.parametrize("tile", [8, 9, 10])
def test_mx_ring_relu_nan(orc, tile):
    """ReLU on the ring maps NaN products (NaN scale, NaN code) to 0 and clips the negatives."""
    api = require_gpu()
    M, N, K = 300, 520, 1024
    say(f"ring relu nan tile={tile}")
    A, SA, B, SB = nonfinite_operands(0, 0, M, N, K, 2100 + tile)
    C = with_tile(tile, lambda: gpu_gemm(api, 0, dev(A), dev(SA), dev(B), dev(SB), M, N, K, flags=api.MXGEMM_RELU))
    ref = orc.mxgemm(0, 0, A, SA, B, SB, M, N, K)
    assert np.isnan(ref[3]).all() and (C[3] == 0).all() and (C[:, 30] == 0).all()
    R = orc.rms_ab(np.nan_to_num(orc.dequant(0, A, SA, M, K)), np.nan_to_num(orc.dequant(0, B, SB, N, K)).T)
    ok, ratio, bad = orc.check(C, orc.relu(ref), K, R)
    assert ok, (ratio, bad)


def test_mx_e5m2_infinity_codes(orc):
    """E5M2 Inf codes (S.11111.00) are infinities: an output with one infinite term is that
    infinity, +Inf + -Inf gives NaN, and Inf times a zero element gives NaN, as in the oracle's
    IEEE fp64 sum. Compared exactly at those outputs and under the bound elsewhere."""
    api = require_gpu()
    M, N, K = 256, 512, 1024
    say("e5m2 infinity codes")
    g = np.random.Generator(np.random.PCG64(1500))

    def codes(shape):   # finite nonzero magnitudes 2^-2 .. 1.75*2^2
        return ((g.integers(0, 2, size=shape) << 7) | (g.integers(13, 18, size=shape) << 2)
                | g.integers(0, 4, size=shape)).astype(np.uint8)
    A, B = codes((M, K)), codes((N, K))
    SA = np.full((M, K // 32), 127, np.uint8)
    SB = np.full((N, K // 32), 127, np.uint8)
    A[1, 100] = 0x7C                     # +Inf in row 1
    A[2, 700] = 0xFC                     # -Inf in row 2
    B[5, 40] = 0x7C                      # +Inf in column 5
    A[2, 40] = 0x40                      # row 2 at K=40: +2, so (2, 5) holds -Inf and +Inf: NaN
    B[9, 100] = 0x00                     # column 9 at K=100: zero, so (1, 9) holds Inf * 0: NaN
    B[5, 700] = 0x3C                     # +1: (2, 5) also holds -Inf * 1
    B[0, 100] = B[0, 700] = 0x3C         # +1: (1, 0) = +Inf, (2, 0) = -Inf
    C = gpu_gemm(api, 1, dev(A), dev(SA), dev(B), dev(SB), M, N, K)
    ref = orc.mxgemm(1, 1, A, SA, B, SB, M, N, K)
    assert np.isnan(ref[2, 5]) and np.isnan(ref[1, 9]) and ref[1, 0] == np.inf and ref[2, 0] == -np.inf
    assert ref[0, 5] in (np.inf, -np.inf)
    R = orc.rms_ab(np.nan_to_num(orc.dequant(1, A, SA, M, K), posinf=0, neginf=0),
                   np.nan_to_num(orc.dequant(1, B, SB, N, K), posinf=0, neginf=0).T)
    ok, ratio, bad = orc.check(C, ref, K, R)
    assert ok, (ratio, bad)


@pytest.mark.parametrize("fmt,M,N,K", [
    (0, 300, 520, 1024), (0, 257, 260, 4096), (0, 1, 4, 1024), (0, 512, 1024, 2048), (0, 33, 1028, 3072),
    (0, 1024, 1024, 1024),
    (4, 300, 520, 1024), (4, 257, 260, 4096), (4, 1, 4, 2048), (4, 512, 1024, 2048), (4, 33, 1028, 3072),
])
def test_mx_pp_ring_every_output(orc, fmt, M, N, K):
    """The 8-wave ping-pong ring (tile 11; K % 1024 == 0): partial tiles in M and N, a single row and
    column strip, one pair of scale groups up to several, and grids of 8 and 16 tiles (XCD remap)."""
    api = require_gpu()
    say(f"pp ring fmt={fmt} M={M} N={N} K={K}")
    C, ref, R = pair_case(orc, api, fmt, fmt, M, N, K, 1600 + M + N + K, tile=11)
    assert not np.isnan(C).any()
    ok, ratio, bad = orc.check(C, ref, K, R)
    assert ok, (ratio, bad)


@pytest.mark.parametrize("fa,fb", [(1, 1), (0, 1), (1, 0)])
@pytest.mark.parametrize("M,N,K", [(300, 520, 1024), (512, 1024, 2048), (33, 1028, 3072), (1, 4, 1024)])
def test_mx_pp_ring_e5m2_pairs(orc, fa, fb, M, N, K):
    """E5M2 with E5M2 or E4M3 on the ping-pong ring (its default where K % 1024 == 0): the MFMA's
    format codes per operand on the E4M3 data path; every output, partial tiles, a grid of 8 tiles,
    a single row."""
    api = require_gpu()
    say(f"pp ring e5m2 fa={fa} fb={fb} M={M} N={N} K={K}")
    p = api.mxgemm_create(M, N, K, fa, fb)
    assert api.mxgemm_plan_info(p)[3] == 4
    api.mxgemm_destroy(p)
    C, ref, R = pair_case(orc, api, fa, fb, M, N, K, 2600 + 7 * fa + 3 * fb + M + N + K, sigma_b=0.02)
    assert not np.isnan(C).any()
    ok, ratio, bad = orc.check(C, ref, K, R)
    assert ok, (ratio, bad)


@pytest.mark.parametrize("fa,fb", [(2, 2), (3, 3), (2, 3), (3, 2)])
@pytest.mark.parametrize("M,N,K", [(300, 520, 1024), (512, 1024, 2048), (33, 1028, 3072), (1, 4, 1024)])
def test_mx_pp_ring_fp6_pairs(orc, fa, fb, M, N, K):
    """FP6 pairs on the ping-pong ring (its default where K % 1024 == 0): 96-byte stage rows copied
    as 12-byte pieces into 16-byte chunks, 24-byte fragments; every output, partial tiles, a grid of
    8 tiles, a single row."""
    api = require_gpu()
    say(f"pp ring fp6 fa={fa} fb={fb} M={M} N={N} K={K}")
    p = api.mxgemm_create(M, N, K, fa, fb)
    assert api.mxgemm_plan_info(p)[3] == 4
    api.mxgemm_destroy(p)
    C, ref, R = pair_case(orc, api, fa, fb, M, N, K, 2800 + 5 * fa + 11 * fb + M + N + K, sigma_b=0.02)
    assert not np.isnan(C).any()
    ok, ratio, bad = orc.check(C, ref, K, R)
    assert ok, (ratio, bad)


def test_mx_pp_ring_fp6_unit_scales_exact(orc):
    """E2M3 x E3M2 on the ping-pong ring at unit scales: E2M3 codes of every value, E3M2 codes with
    exponent fields 0..5 (|b| <= 7), so every product is a multiple of 2^-7 below 53 in magnitude
    and every partial sum over K=1024 is below 2^16, exact in fp32: the GPU must equal the oracle
    after the fp16 rounding."""
    api = require_gpu()
    M, N, K = 300, 520, 1024
    say("pp ring fp6 unit scales exact")
    g = np.random.Generator(np.random.PCG64(2900))

    def pack(codes):
        bits = ((codes[..., None] >> np.arange(6)) & 1).astype(np.uint8).reshape(codes.shape[0], -1)
        return np.ascontiguousarray(np.packbits(bits, axis=1, bitorder="little"))
    ca = g.integers(0, 64, (M, K))
    cb = (g.integers(0, 2, (N, K)) << 5) | (g.integers(0, 6, (N, K)) << 2) | g.integers(0, 4, (N, K))
    SA = np.full((M, K // 32), 127, np.uint8)
    SB = np.full((N, K // 32), 127, np.uint8)
    A, B = pack(ca), pack(cb)
    C = gpu_gemm(api, 2, dev(A), dev(SA), dev(B), dev(SB), M, N, K, fb=3)
    ref = orc.mxgemm(2, 3, A, SA, B, SB, M, N, K)
    assert np.abs(ref).max() < 60000
    assert np.array_equal(C, ref.astype(np.float16).astype(np.float64))


def test_mx_pp_ring_fp6_nonfinite_and_relu(orc):
    """E3M2 x E2M3 on the ping-pong ring with NaN scales, extreme scales, and the ReLU epilogue."""
    api = require_gpu()
    M, N, K = 300, 520, 1024
    say("pp ring fp6 nonfinite")
    A, SA, B, SB = nonfinite_operands(3, 2, M, N, K, 2950)
    C = gpu_gemm(api, 3, dev(A), dev(SA), dev(B), dev(SB), M, N, K, fb=2)
    ref = orc.mxgemm(3, 2, A, SA, B, SB, M, N, K)
    R = orc.rms_ab(np.nan_to_num(orc.dequant(3, A, SA, M, K)), np.nan_to_num(orc.dequant(2, B, SB, N, K)).T)
    ok, ratio, bad = orc.check(C, ref, K, R)
    assert ok, (ratio, bad)
    Cr = gpu_gemm(api, 3, dev(A), dev(SA), dev(B), dev(SB), M, N, K, fb=2, flags=api.MXGEMM_RELU)
    ok, ratio, bad = orc.check(Cr, orc.relu(ref), K, R)
    assert ok, (ratio, bad)


def test_mx_pp_ring_e5m2_nonfinite_and_relu(orc):
    """E5M2 x E4M3 on the ping-pong ring with NaN scales and codes, extreme scales, and ReLU."""
    api = require_gpu()
    M, N, K = 300, 520, 1024
    say("pp ring e5m2 x e4m3 nonfinite")
    A, SA, B, SB = nonfinite_operands(1, 0, M, N, K, 2700)
    C = gpu_gemm(api, 1, dev(A), dev(SA), dev(B), dev(SB), M, N, K, fb=0)
    ref = orc.mxgemm(1, 0, A, SA, B, SB, M, N, K)
    R = orc.rms_ab(np.nan_to_num(orc.dequant(1, A, SA, M, K), posinf=0, neginf=0),
                   np.nan_to_num(orc.dequant(0, B, SB, N, K)).T)
    ok, ratio, bad = orc.check(C, ref, K, R)
    assert ok, (ratio, bad)
    Cr = gpu_gemm(api, 1, dev(A), dev(SA), dev(B), dev(SB), M, N, K, fb=0, flags=api.MXGEMM_RELU)
    ok, ratio, bad = orc.check(Cr, orc.relu(ref), K, R)
    assert ok, (ratio, bad)


@pytest.mark.parametrize("fa,fb", [(0, 4), (1, 4), (4, 0), (4, 1)])
@pytest.mark.parametrize("M,N,K", [(300, 520, 1024), (257, 260, 4096), (512, 1024, 2048), (33, 1028, 3072),
                                   (1, 4, 1024), (256, 8, 5120)])
def test_mx_pp_ring_byte_e2m1_mixes(orc, fa, fb, M, N, K):
    """E4M3 or E5M2 with E2M1, in both orders, on the ping-pong ring (its default where K % 1024 ==
    0): the E2M1 operand's rows staged 128 bytes (four steps) at a time every other slot, 16-byte
    E2M1 fragments; every output, partial tiles, a grid of 8 tiles, a single row, ten scale groups."""
    api = require_gpu()
    say(f"pp ring byte x e2m1 fa={fa} fb={fb} M={M} N={N} K={K}")
    p = api.mxgemm_create(M, N, K, fa, fb)
    assert api.mxgemm_plan_info(p)[3] == 4
    api.mxgemm_destroy(p)
    C, ref, R = pair_case(orc, api, fa, fb, M, N, K, 2900 + 5 * fa + 3 * fb + M + N + K)
    assert not np.isnan(C).any()
    ok, ratio, bad = orc.check(C, ref, K, R)
    assert ok, (ratio, bad)


@pytest.mark.parametrize("fa,fb", [(0, 4), (4, 0)])
def test_mx_pp_ring_byte_e2m1_nonfinite_and_relu(orc, fa, fb):
    """E4M3 x E2M1 in both orders on the ping-pong ring with NaN scales and codes, extreme scales,
    and ReLU; the same operands on the 4-stage ring agree with the oracle too."""
    api = require_gpu()
    M, N, K = 300, 520, 1024
    say(f"pp ring byte x e2m1 nonfinite fa={fa} fb={fb}")
    A, SA, B, SB = nonfinite_operands(fa, fb, M, N, K, 2950 + fa)
    ref = orc.mxgemm(fa, fb, A, SA, B, SB, M, N, K)
    R = orc.rms_ab(np.nan_to_num(orc.dequant(fa, A, SA, M, K)), np.nan_to_num(orc.dequant(fb, B, SB, N, K)).T)
    for tile in (11, 8):
        C = with_tile(tile, lambda: gpu_gemm(api, fa, dev(A), dev(SA), dev(B), dev(SB), M, N, K, fb=fb))
        ok, ratio, bad = orc.check(C, ref, K, R)
        assert ok, (tile, ratio, bad)
    Cr = gpu_gemm(api, fa, dev(A), dev(SA), dev(B), dev(SB), M, N, K, fb=fb, flags=api.MXGEMM_RELU)
    ok, ratio, bad = orc.check(Cr, orc.relu(ref), K, R)
    assert ok, (ratio, bad)


@pytest.mark.parametrize("fmt", [0, 4])
def test_mx_pp_ring_nonfinite_and_relu(orc, fmt):
    """The ping-pong ring with NaN scales and codes, extreme scales, and the ReLU epilogue."""
    api = require_gpu()
    M, N, K = 300, 520, 1024
    say(f"pp ring nonfinite fmt={fmt}")
    A, SA, B, SB = nonfinite_operands(fmt, fmt, M, N, K, 2200 + fmt)
    C = with_tile(11, lambda: gpu_gemm(api, fmt, dev(A), dev(SA), dev(B), dev(SB), M, N, K))
    ref = orc.mxgemm(fmt, fmt, A, SA, B, SB, M, N, K)
    R = orc.rms_ab(np.nan_to_num(orc.dequant(fmt, A, SA, M, K)), np.nan_to_num(orc.dequant(fmt, B, SB, N, K)).T)
    ok, ratio, bad = orc.check(C, ref, K, R)
    assert ok, (ratio, bad)
    Cr = with_tile(11, lambda: gpu_gemm(api, fmt, dev(A), dev(SA), dev(B), dev(SB), M, N, K, flags=api.MXGEMM_RELU))
    ok, ratio, bad = orc.check(Cr, orc.relu(ref), K, R)
    assert ok, (ratio, bad)


# ---- A quantised on load (MXGEMM_QUANT_A): fp16 activations, E4M3 inside the GEMM -------------

def fused_case(orc, api, A16, b_src, M, N, K):
    """C of the fused path (A binary16, quantised on load) and of mx_pack_run(A as fp32) followed by
    the same kernel (tile 11); plus the oracle's C from its own quantisation of the fp32 copy of A."""
    B, SB = gpu_mx_pack(api, 0, b_src)
    plan = api.mxgemm_create(M, N, K, 0, 0, api.MXGEMM_QUANT_A)
    assert api.mxgemm_plan_info(plan)[3] == 4
    Cf = nan_f16((M, N))
    api.mxgemm_run(plan, dev(A16), None, B, SB, Cf)
    plan.close()
    A32 = A16.astype(np.float32)
    A, SA = gpu_mx_pack(api, 0, A32)
    Cu = with_tile(11, lambda: gpu_gemm(api, 0, A, SA, B, SB, M, N, K))
    oA, oSA = orc.mx_quantize(0, A32)
    oB, oSB = orc.mx_quantize(0, b_src)
    assert np.array_equal(host(A), oA) and np.array_equal(host(SA), oSA)
    return host(Cf).astype(np.float64), Cu, (oA, oSA, oB, oSB)


@pytest.mark.parametrize("M,N,K", [(300, 520, 1024), (257, 260, 4096), (1, 4, 1024), (512, 1024, 2048),
                                   (33, 1028, 3072), (1024, 1024, 1024)])
def test_mx_quant_a_fused_equals_pack_then_gemm(orc, M, N, K):
    """Every output of the fused path equals pack + GEMM on the same kernel schedule bit for bit,
    and meets the bound against the oracle."""
    api = require_gpu()
    say(f"quant-A fused M={M} N={N} K={K}")
    A16 = synth.normal((M, K), 1.0, 1700 + M + K).astype(np.float16)
    b_src = synth.normal((N, K), 0.02, 1701 + N + K)
    Cf, Cu, (oA, oSA, oB, oSB) = fused_case(orc, api, A16, b_src, M, N, K)
    assert not np.isnan(Cf).any()
    assert np.array_equal(Cf.astype(np.float16).view(np.uint16), Cu.astype(np.float16).view(np.uint16))
    ref = orc.mxgemm(0, 0, oA, oSA, oB, oSB, M, N, K)
    R = orc.rms_ab(orc.dequant(0, oA, oSA, M, K), orc.dequant(0, oB, oSB, N, K).T)
    ok, ratio, bad = orc.check(Cf, ref, K, R)
    assert ok, (ratio, bad)


def test_mx_quant_a_fused_edge_values(orc):
    """fp16 blocks at the edges of the quantiser: all-zero and -0 blocks, subnormal fp16 blocks, the
    largest fp16 values, exact ties of the E4M3 grid, values that saturate (scaled above 464), and
    blocks holding Inf or NaN (their rows of C are NaN). Fused equals pack + GEMM bit for bit
    (NaN positions included) and meets the bound on the finite outputs."""
    api = require_gpu()
    M, N, K = 96, 260, 1024
    say("quant-A fused edge values")
    A = synth.normal((M, K), 1.0, 1800).astype(np.float32)
    A[0] = 0.0
    A[1, :64] = -0.0
    A[2] *= np.float32(2.0 ** -20)                    # fp16 subnormals and tiny normals
    A[3, 32:64] = np.float32(2.0 ** -24) * np.arange(1, 33, dtype=np.float32)
    A[4] = np.sign(A[4]) * np.float32(65504.0)        # the largest fp16
    grid = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    mids = (grid[:-1] + grid[1:]) / 2
    A[5, :32] = np.float32(448.0)                     # amax 448: scale 2^0, ties of the grid
    A[5, 1:32] = mids[np.linspace(0, len(mids) - 1, 31).astype(int)]
    A[6, :32] = np.float32(500.0)                     # amax 500: scale 2^0, 500 -> 448 (saturates)
    A[6, 1:32] = np.float32(470.0)
    A[7, 100] = np.inf
    A[8, 500] = np.nan
    A[9, 33] = -np.inf
    A16 = A.astype(np.float16)
    b_src = synth.normal((N, K), 0.02, 1801)
    Cf, Cu, (oA, oSA, oB, oSB) = fused_case(orc, api, A16, b_src, M, N, K)
    assert np.isnan(Cf[7]).all() and np.isnan(Cf[8]).all() and np.isnan(Cf[9]).all()
    assert not np.isnan(np.delete(Cf, [7, 8, 9], axis=0)).any()
    assert np.array_equal(Cf.astype(np.float16).view(np.uint16), Cu.astype(np.float16).view(np.uint16))
    ref = orc.mxgemm(0, 0, oA, oSA, oB, oSB, M, N, K)
    R = orc.rms_ab(np.nan_to_num(orc.dequant(0, oA, oSA, M, K)), orc.dequant(0, oB, oSB, N, K).T)
    ok, ratio, bad = orc.check(Cf, ref, K, R)
    assert ok, (ratio, bad)


def test_mx_quant_a_fused_prefill_every_output(orc):
    """The prefill shape (M=2048, N=14336, K=4096, fp16 activations N(0,1), weights 0.02 N(0,1)):
    the fused path equals pack + GEMM on every output, bit for bit, and sampled outputs meet the
    bound against the oracle."""
    api = require_gpu()
    M, N, K = 2048, 14336, 4096
    say("quant-A fused prefill")
    A16 = synth.normal((M, K), 1.0, synth.seed_for(synth.MXFP8_PREFILL, 0)).astype(np.float16)
    b_src = synth.normal((N, K), 0.02, synth.seed_for(synth.MXFP8_PREFILL, 1))
    B, SB = gpu_mx_pack(api, 0, b_src)
    plan = api.mxgemm_create(M, N, K, 0, 0, api.MXGEMM_QUANT_A)
    Cf = nan_f16((M, N))
    api.mxgemm_run(plan, dev(A16), None, B, SB, Cf)
    plan.close()
    A, SA = gpu_mx_pack(api, 0, A16.astype(np.float32))
    pu = api.mxgemm_create(M, N, K, 0, 0)
    Cu = nan_f16((M, N))
    api.mxgemm_run(pu, A, SA, B, SB, Cu)
    pu.close()
    cf, cu = host(Cf), host(Cu)
    assert np.isfinite(cf).all()
    assert np.array_equal(cf.view(np.uint16), cu.view(np.uint16))
    oA, oSA = orc.mx_quantize(0, A16.astype(np.float32))
    oB, oSB = orc.mx_quantize(0, b_src)
    ms, ns = synth.sample_points(M, N, 2048, 97)
    ref = orc.mxgemm_points(0, 0, oA, oSA, oB, oSB, K, ms, ns)
    ok, ratio, bad = orc.check(cf[ms, ns].astype(np.float64), ref, K, R_of(orc, 0, oA, oSA, oB, oSB, M, N, K))
    say(f"quant-A prefill: worst err/bound {ratio:.3f}")
    assert ok, (ratio, bad)


def test_mx_quant_a_fused_relu(orc):
    api = require_gpu()
    M, N, K = 300, 520, 1024
    say("quant-A fused relu")
    A16 = synth.normal((M, K), 1.0, 1900).astype(np.float16)
    b_src = synth.normal((N, K), 1.0, 1901)
    B, SB = gpu_mx_pack(api, 0, b_src)
    plan = api.mxgemm_create(M, N, K, 0, 0, api.MXGEMM_QUANT_A | api.MXGEMM_RELU)
    C = nan_f16((M, N))
    api.mxgemm_run(plan, dev(A16), None, B, SB, C)
    plan.close()
    oA, oSA = orc.mx_quantize(0, A16.astype(np.float32))
    oB, oSB = orc.mx_quantize(0, b_src)
    ref = orc.relu(orc.mxgemm(0, 0, oA, oSA, oB, oSB, M, N, K))
    got = host(C).astype(np.float64)
    assert (got >= 0).all()
    ok, ratio, bad = orc.check(got, ref, K, R_of(orc, 0, oA, oSA, oB, oSB, M, N, K))
    assert ok, (ratio, bad)
