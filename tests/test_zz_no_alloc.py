"""mxmatvec_run_noalloc (the split matvec's workspace in the library's static scratch array) against
mxmatvec_run with a caller workspace: the same kernels, so the same bits, and both within the
acceptance bound of the oracle. Two calls in a row, the second on a smaller problem, so the second
runs on the scratch contents the first left behind."""
import numpy as np
import pytest
import torch

from block_scaled_quantized_amd import synth
from gpu_common import dev, gpu_int_pack, host, nan_f16, require_gpu, say

pytestmark = pytest.mark.gpu


def one(orc, api, fw, M, K, N, seed):
    w = synth.normal((K, N), 0.02, seed)
    x = synth.normal((M, K), 1.0, seed + 1).astype(np.float16)
    W, Ws = gpu_int_pack(api, fw, w)
    need = api.mxmatvec_workspace_size(M, N, K, fw)
    assert 0 < need <= api.MXMATVEC_SCRATCH_BYTES
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    xd = dev(x)
    y_ws = nan_f16((M, N))
    api.mxmatvec_run(M, N, K, xd, W, fw, Ws, y_ws, ws)
    y_na = nan_f16((M, N))
    api.mxmatvec_run_noalloc(M, N, K, xd, W, fw, Ws, y_na)
    a, b = host(y_ws), host(y_na)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), "noalloc differs from the workspace call"
    q, s = orc.int_quantize(fw, w)
    oW = q.view(np.uint8) if fw == api.MX_INT8 else orc.pack_int4(q)
    ok, ratio, bad = orc.check(b.astype(np.float64), orc.matvec(fw, x, oW, s, K, N), K,
                               orc.rms_ab(x.astype(np.float64), orc.dequant(fw, oW, s, K, N)))
    say(f"noalloc fw={fw} M={M} K={K} N={N}: worst err/bound {ratio:.3f}")
    assert ok, (ratio, bad)


def test_noalloc_matches_workspace_call_twice(orc):
    api = require_gpu()
    say("noalloc: decode shape, then a smaller one")
    one(orc, api, api.MX_INT4, 8, 4096, 14336, 4100)     # the largest decode workload (int4, S = 9)
    one(orc, api, api.MX_INT8, 3, 1024, 4128, 4200)      # smaller, on the scratch the first left


def test_noalloc_small_m_gemm_split_twice(orc):
    """The small-M GEMM with K split across workgroups (partials and counters in the scratch
    array): the same bits as the workspace call, then a smaller problem on what the first left."""
    api = require_gpu()
    say("noalloc: small-M GEMM split, then a smaller one")
    one(orc, api, api.MX_INT8, 64, 1024, 4096, 4400)     # 64 tiles, K split 4 ways
    one(orc, api, api.MX_INT4, 24, 2048, 1056, 4500)     # 9 tiles, K split 8 ways


def test_noalloc_small_m_gemm_block_runs_twice(orc):
    """The small-M GEMM with block runs over 64 x 128 tiles (partial tiles and counters in the
    scratch array), then a K split on what it left: the same bits as the workspace call."""
    api = require_gpu()
    say("noalloc: small-M GEMM block runs, then a K split")
    one(orc, api, api.MX_INT4, 160, 1024, 12288, 4600)   # 288 tiles, runs of 36 blocks
    one(orc, api, api.MX_INT8, 64, 1024, 4096, 4700)     # 64 tiles, K split 4 ways


def test_noalloc_small_m_gemm_and_single_pass(orc):
    """Shapes that need no workspace (a small-M GEMM whose K is too short to split, and a decode
    shape the split kernel does not take): same bits as mxmatvec_run."""
    api = require_gpu()
    for fw, M, K, N in ((api.MX_INT8, 64, 224, 4096), (api.MX_INT4, 2, 64, 96)):
        say(f"noalloc passthrough fw={fw} M={M} K={K} N={N}")
        assert api.mxmatvec_workspace_size(M, N, K, fw) == 0
        w = synth.normal((K, N), 0.02, 4300 + M)
        x = synth.normal((M, K), 1.0, 4301 + M).astype(np.float16)
        W, Ws = gpu_int_pack(api, fw, w)
        xd = dev(x)
        y1, y2 = nan_f16((M, N)), nan_f16((M, N))
        api.mxmatvec_run(M, N, K, xd, W, fw, Ws, y1)
        api.mxmatvec_run_noalloc(M, N, K, xd, W, fw, Ws, y2)
        assert np.array_equal(host(y1).view(np.uint16), host(y2).view(np.uint16))
        assert not np.isnan(host(y2)).any()
