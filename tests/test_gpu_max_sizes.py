"""The largest problems the API accepts along each axis, against the oracle.

M, N and K go up to MX_MAX_DIM (2^20). Each case takes one axis to the limit, or far enough that an
operand passes 2^31 bytes, so any 32-bit byte offset in a kernel's addressing would overflow. The
other axes stay small, so the oracle can check the outputs (all of them, or samples that include
the first and last tiles and the rows or columns around the 2^31-byte mark).

A 4 GiB operand is drawn as E4M3 codes of +-1 with random signs and unit scales. Every row is
then distinct, so a wrong row offset would change C, and every element squares to 1. The R of
the acceptance bound therefore equals the oracle's rms_ab on a single row, with no 4 GiB host copy.
"""
import os

import numpy as np
import pytest
import torch

from block_scaled_quantized_amd import synth
from gpu_common import dev, gpu_gemm, gpu_int_pack, gpu_mx_pack, host, nan_f16, require_gpu, say

pytestmark = pytest.mark.gpu

E4M3_ONE = 0x38


def pm1_codes_to_gpu(rows, K, seed, keep_rows):
    """E4M3 codes +-1 [rows][K] drawn in chunks straight into device memory; returns the device
    tensor and the host copies of the rows in keep_rows (in that order)."""
    out = torch.empty((rows, K), dtype=torch.uint8, device="cuda")
    kept = np.empty((len(keep_rows), K), dtype=np.uint8)
    keep = np.asarray(keep_rows)
    step = max(1, (256 << 20) // K)
    for c, r0 in enumerate(range(0, rows, step)):
        r1 = min(rows, r0 + step)
        sign = synth.random_bytes((r1 - r0, K), seed + c) & np.uint8(0x80)
        chunk = sign | np.uint8(E4M3_ONE)
        out[r0:r1] = torch.from_numpy(chunk).cuda()
        sel = np.nonzero((keep >= r0) & (keep < r1))[0]
        kept[sel] = chunk[keep[sel] - r0]
    torch.cuda.synchronize()
    return out, kept


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


def sample_rows(M, extra):
    rows = {0, 1, 255, 256, M - 257, M - 256, M - 1, *extra}
    rng = synth.rng(77)
    rows |= set(int(r) for r in rng.integers(0, M, 200))
    return np.array(sorted(rows), dtype=np.int64)


def test_mx_gemm_max_rows(orc):
    """M = 2^20 rows of K = 4096 E4M3 codes: A is 4 GiB, so row offsets pass 2^31 bytes from row
    2^19 on. Default kernel, the 4-stage ring and the 64x64 fallback."""
    api = require_gpu()
    M, N, K = 1 << 20, 4, 4096      # M = MX_MAX_DIM
    say(f"max rows: E4M3 {M}x{N}x{K}")
    ms_all = sample_rows(M, [(1 << 19) - 1, 1 << 19, (1 << 19) + 1])
    A, A_rows = pm1_codes_to_gpu(M, K, 9100, ms_all)
    SA = torch.full((M, K // 32), 127, dtype=torch.uint8, device="cuda")
    B, SB = gpu_mx_pack(api, api.MX_E4M3, synth.normal((N, K), 1.0, 9101))
    oB, oSB = host(B), host(SB)
    sa = np.full((len(ms_all), K // 32), 127, dtype=np.uint8)
    ms = np.repeat(np.arange(len(ms_all)), N)
    ns = np.tile(np.arange(N), len(ms_all))
    ref = orc.mxgemm_points(api.MX_E4M3, api.MX_E4M3, A_rows, sa, oB, oSB, K, ms, ns)
    R = orc.rms_ab(orc.dequant(api.MX_E4M3, A_rows[:1], sa[:1], 1, K), orc.dequant(api.MX_E4M3, oB, oSB, N, K).T)
    for tile in (None, 8, 3):
        C = with_tile(tile, lambda: gpu_gemm(api, api.MX_E4M3, A, SA, B, SB, M, N, K))
        assert np.isfinite(C).all(), f"tile {tile}: an output left unwritten"
        ok, ratio, bad = orc.check(C[ms_all][ms, ns], ref, K, R)
        say(f"max rows tile {tile}: worst err/bound {ratio:.3f}")
        assert ok, (tile, ratio, bad)
    del A, SA


def test_mx_gemm_max_columns(orc):
    """N = 2^20 columns of K = 4096 E4M3 codes: B is 4 GiB, so column offsets pass 2^31 bytes from
    column 2^19 on. Default kernel, the 4-stage ring and the 64x64 fallback."""
    api = require_gpu()
    M, N, K = 4, 1 << 20, 4096
    say(f"max columns: E4M3 {M}x{N}x{K}")
    ns_all = sample_rows(N, [(1 << 19) - 1, 1 << 19, (1 << 19) + 1])
    B, B_rows = pm1_codes_to_gpu(N, K, 9200, ns_all)
    SB = torch.full((N, K // 32), 127, dtype=torch.uint8, device="cuda")
    A, SA = gpu_mx_pack(api, api.MX_E4M3, synth.normal((M, K), 1.0, 9201))
    oA, oSA = host(A), host(SA)
    sb = np.full((len(ns_all), K // 32), 127, dtype=np.uint8)
    ms = np.repeat(np.arange(M), len(ns_all))
    ns = np.tile(np.arange(len(ns_all)), M)
    ref = orc.mxgemm_points(api.MX_E4M3, api.MX_E4M3, oA, oSA, B_rows, sb, K, ms, ns)
    R = orc.rms_ab(orc.dequant(api.MX_E4M3, oA, oSA, M, K), orc.dequant(api.MX_E4M3, B_rows[:1], sb[:1], 1, K).T)
    for tile in (None, 8, 3):
        C = with_tile(tile, lambda: gpu_gemm(api, api.MX_E4M3, A, SA, B, SB, M, N, K))
        assert np.isfinite(C).all(), f"tile {tile}: an output left unwritten"
        ok, ratio, bad = orc.check(C[:, ns_all][ms, ns], ref, K, R)
        say(f"max columns tile {tile}: worst err/bound {ratio:.3f}")
        assert ok, (tile, ratio, bad)
    del B, SB


def test_gemm_max_k(orc):
    """K = 2^20: MXFP8 (the ping-pong kernel's 16384 steps in one tile) and fp16 (ping-pong and the
    64x64 fallback), every output against the oracle."""
    api = require_gpu()
    K = 1 << 20
    M, N = 5, 12
    say(f"max K: E4M3 {M}x{N}x{K}")
    a_src = synth.normal((M, K), 1.0, 9300)
    b_src = synth.normal((N, K), 1.0, 9301)
    A, SA = gpu_mx_pack(api, api.MX_E4M3, a_src)
    B, SB = gpu_mx_pack(api, api.MX_E4M3, b_src)
    oA, oSA = orc.mx_quantize(api.MX_E4M3, a_src)
    oB, oSB = orc.mx_quantize(api.MX_E4M3, b_src)
    assert np.array_equal(host(A), oA) and np.array_equal(host(B), oB)
    C = gpu_gemm(api, api.MX_E4M3, A, SA, B, SB, M, N, K)
    ref = orc.mxgemm(api.MX_E4M3, api.MX_E4M3, oA, oSA, oB, oSB, M, N, K)
    R = orc.rms_ab(orc.dequant(api.MX_E4M3, oA, oSA, M, K), orc.dequant(api.MX_E4M3, oB, oSB, N, K).T)
    ok, ratio, bad = orc.check(C, ref, K, R)
    say(f"max K E4M3: worst err/bound {ratio:.3f}")
    assert ok, (ratio, bad)

    M, N = 17, 8
    say(f"max K: fp16 {M}x{N}x{K}")
    A16 = synth.uniform_pm1((M, K), 9310).astype(np.float16)
    B16 = synth.uniform_pm1((K, N), 9311).astype(np.float16)
    ref = orc.gemm_f16(A16, B16)
    R = orc.rms_ab(A16.astype(np.float64), B16.astype(np.float64))
    for tile in (None, 3):
        C = with_tile(tile, lambda: gpu_gemm(api, api.MX_F16, dev(A16), None, dev(B16), None, M, N, K))
        ok, ratio, bad = orc.check(C, ref, K, R)
        say(f"max K fp16 tile {tile}: worst err/bound {ratio:.3f}")
        assert ok, (tile, ratio, bad)


def matvec_case(orc, api, fw, M, K, N, seed, workspace):
    w = synth.normal((K, N), 0.02, seed)
    x = synth.normal((M, K), 1.0, seed + 1).astype(np.float16)
    W, Ws = gpu_int_pack(api, fw, w)
    q, s = orc.int_quantize(fw, w)
    del w
    oW = q.view(np.uint8) if fw == api.MX_INT8 else orc.pack_int4(q)
    assert np.array_equal(host(W), oW) and np.array_equal(host(Ws).view(np.uint16), s.view(np.uint16))
    need = api.mxmatvec_workspace_size(M, N, K, fw)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device="cuda") if workspace else None
    y = nan_f16((M, N))
    api.mxmatvec_run(M, N, K, dev(x), W, fw, Ws, y, ws)
    out = host(y).astype(np.float64)
    ref = orc.matvec(fw, x, oW, s, K, N)
    R = orc.rms_ab(x.astype(np.float64), orc.dequant(fw, oW, s, K, N))
    ok, ratio, bad = orc.check(out, ref, K, R)
    say(f"matvec fw={fw} M={M} K={K} N={N} workspace={workspace} (need {need}): worst err/bound {ratio:.3f}")
    assert ok, (ratio, bad)


def test_matvec_max_n(orc):
    """N = 2^20 columns (int8 and int4), every output against the oracle."""
    api = require_gpu()
    N = 1 << 20
    matvec_case(orc, api, api.MX_INT8, 8, 64, N, 9400, True)
    matvec_case(orc, api, api.MX_INT4, 1, 64, N, 9410, False)


def test_matvec_max_k(orc):
    """K = 2^20 rows of weights: the decode matvec and the small-M GEMM (with and without a
    workspace), every output against the oracle."""
    api = require_gpu()
    K = 1 << 20
    matvec_case(orc, api, api.MX_INT4, 3, K, 32, 9500, True)
    matvec_case(orc, api, api.MX_INT8, 40, K, 32, 9510, True)
    matvec_case(orc, api, api.MX_INT8, 40, K, 32, 9520, False)


def test_codecs_max_columns(orc):
    """Pack and unpack of rows 2^20 elements long: codes and scales bit for bit with the oracle's
    quantiser, and the unpacked values bit for bit with the oracle's decoders."""
    api = require_gpu()
    cols = 1 << 20
    src = synth.normal((2, cols), 1.0, 9600)
    say(f"codecs: E4M3 2x{cols}")
    codes, scales = gpu_mx_pack(api, api.MX_E4M3, src)
    oc, os_ = orc.mx_quantize(api.MX_E4M3, src)
    assert np.array_equal(host(codes), oc) and np.array_equal(host(scales), os_)
    out = torch.full((2, cols), 12345.678, dtype=torch.float32, device="cuda")
    api.mx_unpack_run(api.MX_E4M3, codes, scales, 2, cols, out)
    want = orc.dequant(api.MX_E4M3, oc, os_, 2, cols).astype(np.float32)
    got = host(out)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
