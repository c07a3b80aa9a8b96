"""GPU int8/int4 dequant matvec against the oracle.

Weights W [K][N] are drawn 0.02*N(0,1) and quantised by the GPU codec (checked bit-exact against
the oracle's quantiser first); x is fp16 from N(0,1). Every output is compared with the oracle's
fp64 block formula under |y - y_ref| <= 2^-10 |y_ref| + 1e-3 sqrt(K) R, R the rms of |x_mk w_kn|
over the dequantised weights. Both paths run: K split across workgroups and unsplit (no
workspace). The split path shares one workspace, zeroed once, across every case in this file, so
each case also checks that the calls before it left the workspace's counters at zero. Each case
calls it three times: on x, then on different activations x2 (checked against the oracle too, so a
strip whose partial sums or counter were left stale by the first call shows up), then on x again,
which must reproduce the first result bit for bit. Every output buffer is filled with NaN before
each call, so an output a kernel fails to write cannot pass.
"""
import numpy as np
import pytest
import torch

from block_scaled_quantized_amd import synth
from gpu_common import dev, empty, gpu_int_pack, host, nan_f16, require_gpu, say

pytestmark = pytest.mark.gpu


_WS = {}


def workspace(api, M, N, K, fw):
    """The shared workspace, zeroed once (and again only when it must grow)."""
    need = api.mxmatvec_workspace_size(M, N, K, fw)
    if need == 0:
        return None
    if _WS.get("buf") is None or _WS["buf"].numel() < need:
        _WS["buf"] = torch.zeros(max(need, 8 << 20), dtype=torch.uint8, device="cuda")
    return _WS["buf"]


def run_case(orc, api, fw, M, K, N, seed_w, seed_x, path="split"):
    w = synth.normal((K, N), 0.02, seed_w)
    x = synth.normal((8, K), 1.0, seed_x).astype(np.float16)[:M]
    x2 = synth.normal((8, K), 1.0, seed_x + 5000).astype(np.float16)[:M]
    W, Ws = gpu_int_pack(api, fw, w)
    q, s = orc.int_quantize(fw, w)
    oW = q.view(np.uint8) if fw == api.MX_INT8 else orc.pack_int4(q)
    assert np.array_equal(host(W), oW) and np.array_equal(host(Ws).view(np.uint16), s.view(np.uint16))
    ws = workspace(api, M, N, K, fw) if path == "split" else None
    wdeq = orc.dequant(fw, oW, s, K, N)
    worst, nbad, all_ok = 0.0, 0, True
    first = None
    for xi in (x, x2, x):
        y = nan_f16((M, N))
        api.mxmatvec_run(M, N, K, dev(xi), W, fw, Ws, y, ws)
        got16 = host(y).copy()
        if first is None:
            first = got16
        elif xi is x:         # the third call: the first call's bits again
            assert np.array_equal(got16.view(np.uint16), first.view(np.uint16)), "matvec not repeatable"
            continue
        ok, ratio, bad = orc.check(got16.astype(np.float64), orc.matvec(fw, xi, oW, s, K, N), K,
                                   orc.rms_ab(xi.astype(np.float64), wdeq))
        all_ok, worst, nbad = all_ok and ok, max(worst, ratio), nbad + bad
    return all_ok, worst, nbad


@pytest.mark.parametrize("path", ["split", "single"])
@pytest.mark.parametrize("fw", [32, 33])
@pytest.mark.parametrize("M", [1, 8])
def test_matvec_decode_shape_full(orc, fw, M, path):
    """K=4096, N=14336 at M=1 and M=8: every output."""
    api = require_gpu()
    say(f"matvec fw={fw} M={M} full size path={path}")
    ok, ratio, bad = run_case(orc, api, fw, M, 4096, 14336, synth.seed_for(synth.MATVEC, 1),
                              synth.seed_for(synth.MATVEC, 0), path)
    say(f"worst err/bound {ratio:.3f}")
    assert ok, (ratio, bad)


@pytest.mark.parametrize("path", ["split", "single"])
@pytest.mark.parametrize("fw", [32, 33])
@pytest.mark.parametrize("M,K,N", [(1, 32, 32), (2, 64, 96), (3, 96, 160), (5, 4096, 64), (7, 1024, 1056),
                                   (8, 160, 4128), (4, 8192, 512), (6, 544, 14336), (8, 32768, 96),
                                   (1, 1024, 32768)])
def test_matvec_ragged(orc, fw, M, K, N, path):
    api = require_gpu()
    say(f"matvec fw={fw} M={M} K={K} N={N} path={path}")
    ok, ratio, bad = run_case(orc, api, fw, M, K, N, 7 * K + N, 3 * M + K, path)
    assert ok, (ratio, bad)


def test_matvec_zero_block_and_repeat(orc):
    """An all-zero weight block (scale 0) and two calls in a row on the same output buffer."""
    api = require_gpu()
    say("matvec zero block + repeat")
    M, K, N = 4, 128, 64
    w = synth.normal((K, N), 0.02, 3)
    w[32:64, :] = 0.0
    x = synth.normal((M, K), 1.0, 4).astype(np.float16)
    W, Ws = gpu_int_pack(api, api.MX_INT8, w)
    y = nan_f16((M, N))
    api.mxmatvec_run(M, N, K, dev(x), W, api.MX_INT8, Ws, y)
    first = host(y).copy()
    y = nan_f16((M, N))
    api.mxmatvec_run(M, N, K, dev(x), W, api.MX_INT8, Ws, y)
    assert np.array_equal(first.view(np.uint16), host(y).view(np.uint16))     # deterministic
    q, s = orc.int_quantize(api.MX_INT8, w)
    ref = orc.matvec(api.MX_INT8, x, q.view(np.uint8), s, K, N)
    ok, ratio, bad = orc.check(first.astype(np.float64), ref, K,
                               orc.rms_ab(x.astype(np.float64), orc.dequant(32, q.view(np.uint8), s, K, N)))
    assert ok, (ratio, bad)


def test_matvec_small_workspace_falls_back(orc):
    """A workspace below the requirement runs the single-pass kernel: still within the bound."""
    api = require_gpu()
    M, K, N = 8, 4096, 1024
    need = api.mxmatvec_workspace_size(M, N, K, api.MX_INT8)
    say(f"matvec small workspace need={need}")
    assert need > 0
    w = synth.normal((K, N), 0.02, 11)
    x = synth.normal((M, K), 1.0, 12).astype(np.float16)
    W, Ws = gpu_int_pack(api, api.MX_INT8, w)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    y = nan_f16((M, N))
    api.mxmatvec_run(M, N, K, dev(x), W, api.MX_INT8, Ws, y, ws, need - 16)
    q, s = orc.int_quantize(api.MX_INT8, w)
    ref = orc.matvec(api.MX_INT8, x, q.view(np.uint8), s, K, N)
    R = orc.rms_ab(x.astype(np.float64), orc.dequant(32, q.view(np.uint8), s, K, N))
    ok, ratio, bad = orc.check(host(y).astype(np.float64), ref, K, R)
    assert ok, (ratio, bad)
    assert int(ws.sum().item()) == 0      # untouched


# ---- the same product at 9 <= M <= 256 (small-M GEMM kernel) --------------------------------

def wq_case(orc, api, fw, M, K, N, seed_w, seed_x, path):
    """path "split": with the shared workspace (K split across workgroups where the plan asks for a
    workspace), called on x, on x2 (checked too, so stale partials or counters show up) and on x
    again (the same bits); "single": no workspace. Returns x, the codes and scales, y from x, R."""
    w = synth.normal((K, N), 0.02, seed_w)
    x = synth.normal((M, K), 1.0, seed_x).astype(np.float16)
    x2 = synth.normal((M, K), 1.0, seed_x + 7000).astype(np.float16)
    W, Ws = gpu_int_pack(api, fw, w)
    q, s = orc.int_quantize(fw, w)
    oW = q.view(np.uint8) if fw == api.MX_INT8 else orc.pack_int4(q)
    assert np.array_equal(host(W), oW) and np.array_equal(host(Ws).view(np.uint16), s.view(np.uint16))
    R = orc.rms_ab(x.astype(np.float64), orc.dequant(fw, oW, s, K, N))
    if path == "single":
        y = nan_f16((M, N))
        api.mxmatvec_run(M, N, K, dev(x), W, fw, Ws, y)
        return x, oW, s, host(y).astype(np.float64), R
    ws = workspace(api, M, N, K, fw)
    outs = []
    for xi in (x, x2, x):
        y = nan_f16((M, N))
        api.mxmatvec_run(M, N, K, dev(xi), W, fw, Ws, y, ws)
        outs.append(host(y).copy())
    assert np.array_equal(outs[0].view(np.uint16), outs[2].view(np.uint16)), "small-M GEMM not repeatable"
    R2 = orc.rms_ab(x2.astype(np.float64), orc.dequant(fw, oW, s, K, N))
    ok, ratio, bad = orc.check(outs[1].astype(np.float64), orc.matvec(fw, x2, oW, s, K, N), K, R2)
    assert ok, ("second activations", ratio, bad)
    return x, oW, s, outs[0].astype(np.float64), R


def wq_splits(M, K, N):
    """The K split the plan takes with a workspace: 128-column strips, 32-row tiles, about 256
    workgroups, at most 8 splits and at least 8 blocks each (1: not split)."""
    tiles = -(-N // 128) * -(-M // 32)
    S = min(256 // tiles, 8, K // 256)
    return S if S >= 2 else 1


def wq_runs(M, K, N):
    """Blocks per run where the plan deals out the blocks of the 64 x 128 tiles in equal runs to 256
    workgroups (more than 256 tiles filling less than 90% of their rounds, runs of 8 blocks or
    more; 0: whole tiles)."""
    if wq_splits(M, K, N) > 1 or M <= 32:
        return 0
    T = -(-N // 128) * -(-M // 64)
    rounds = -(-T // 256)
    if T < 192 or rounds < 2 or T * 10 >= rounds * 256 * 9:
        return 0
    QB = -(-T * (K // 32) // 256)
    return QB if QB >= 8 else 0


@pytest.mark.parametrize("path", ["split", "single"])
@pytest.mark.parametrize("fw", [32, 33])
@pytest.mark.parametrize("M,K,N", [(9, 32, 32), (16, 1024, 1056), (31, 96, 160), (33, 4096, 64), (64, 544, 4128),
                                   (100, 256, 12288), (128, 4096, 512), (129, 160, 96), (200, 1024, 1024),
                                   (256, 2048, 320), (150, 96, 12800), (200, 64, 16384), (129, 64, 19200),
                                   (20, 64, 25600), (144, 96, 6144), (24, 2048, 1056), (17, 512, 14336),
                                   (160, 1024, 12288), (150, 3104, 12192), (256, 1024, 16512), (40, 512, 102400)])
def test_wq_gemm_ragged(orc, fw, M, K, N, path):
    """Every output: partial row tiles, partial column strips, one block of K up to many. Unsplit
    launch shapes: 128-column strips with 64-row tiles at M=100/N=12288, M=150/N=12800,
    M=200/N=16384 and M=129/N=19200 (the last tile with 1 row); 64-column strips with 32-row tiles at
    M=20/N=25600 and M=144/N=6144; 64-column strips with 16-row tiles for the rest. With a workspace,
    K is split 4 ways at M=16/N=1056 and M=200/N=1024, 8 ways at M=33/N=64, M=128/N=512,
    M=256/N=320 and M=24/N=1056, and 2 ways at M=64/K=544 (17 blocks: 8 + 9) and M=17/N=14336.
    With a workspace, block runs over 64 x 128 tiles at M=160/N=12288 (288 tiles), M=150/N=12192/
    K=3104 (a 22-row last row tile, a 32-column last strip, 97 blocks per tile, runs of 110),
    M=256/N=16512 (516 tiles) and M=40/N=102400 (800 tiles of 40 rows): runs that end inside a tile,
    tiles shared by two runs and tiles wholly inside one."""
    api = require_gpu()
    S, QB = wq_splits(M, K, N), wq_runs(M, K, N)
    need = api.mxmatvec_workspace_size(M, N, K, fw)
    assert (need > 0) == (S > 1 or QB > 0)
    if S > 1:
        assert need == 16384 + -(-(S * M * N * 4) // 256) * 256
    if QB > 0:
        T = -(-N // 128) * -(-M // 64)
        assert need == 16384 + -(-T * (K // 32) // QB) * 2 * 64 * 128 * 4
    say(f"wq gemm fw={fw} M={M} K={K} N={N} path={path} splits={S if path == 'split' else 1} "
        f"runs={QB if path == 'split' else 0}")
    x, oW, s, got, R = wq_case(orc, api, fw, M, K, N, 13 * K + N + M, 5 * K + M, path)
    ok, ratio, bad = orc.check(got, orc.matvec(fw, x, oW, s, K, N), K, R)
    assert ok, (ratio, bad)


@pytest.mark.parametrize("path", ["split", "single"])
@pytest.mark.parametrize("fw", [32, 33])
@pytest.mark.parametrize("M,K,N", [(128, 4096, 12288), (64, 4096, 4096), (256, 4096, 12288)])
def test_wq_gemm_full_size_sampled(orc, fw, M, K, N, path):
    """The W8A16 / W4A16 prefill shapes: 2048 sampled outputs (corners included) against the
    oracle's per-element formula, and every output written (y starts as NaN). M=64/N=4096 splits K
    4 ways with a workspace; M=128/N=12288 is never split; M=256/N=12288 (384 tiles) takes block
    runs of 192 blocks with a workspace."""
    api = require_gpu()
    say(f"wq gemm full fw={fw} M={M} K={K} N={N} path={path}")
    x, oW, s, got, R = wq_case(orc, api, fw, M, K, N, synth.seed_for(synth.WQ_PREFILL, 1),
                                synth.seed_for(synth.WQ_PREFILL, 0), path)
    assert np.isfinite(got).all()
    ms, ns = synth.sample_points(M, N, 2048, 77)
    ref = np.array([orc.matvec_elem(fw, x, oW, s, K, N, int(m), int(n)) for m, n in zip(ms, ns)])
    ok, ratio, bad = orc.check(got[ms, ns], ref, K, R)
    say(f"worst err/bound {ratio:.3f}")
    assert ok, (ratio, bad)
