"""Calls queued on several streams at once, and calls captured in a HIP graph (through
torch.cuda.graph) and replayed: every result equals, bit for bit, the same call made alone.

The header promises both. GPU entry points only queue work on their stream, a plan holds host
metadata only and may be used from several streams at once, and the matvec's workspace (or the
no-alloc scratch array) has its counters back at zero after every call, so a captured call can be
replayed. Each graph replay runs after eager calls on the same buffers and the outputs are
NaN-filled before it, so a replay that skipped work or read stale counters would show.
"""
import numpy as np
import pytest
import torch

from block_scaled_quantized_amd import synth
from gpu_common import dev, gpu_int_pack, gpu_mx_pack, host, nan_f16, require_gpu, say

pytestmark = pytest.mark.gpu


def bits(t: torch.Tensor) -> np.ndarray:
    return host(t).view(np.uint16)


def mx_operands(api, fmt, M, N, K, seed):
    A, SA = gpu_mx_pack(api, fmt, synth.normal((M, K), 1.0, seed))
    B, SB = gpu_mx_pack(api, fmt, synth.normal((N, K), 0.02, seed + 1))   # B stored [N][K]
    return A, SA, B, SB


def int_operands(api, fw, M, K, N, seed):
    W, Ws = gpu_int_pack(api, fw, synth.normal((K, N), 0.02, seed))
    x = dev(synth.normal((M, K), 1.0, seed + 1).astype(np.float16))
    return x, W, Ws


def test_one_plan_two_streams(monkeypatch):
    """One MXFP8 plan used on two streams at once (calls alternating, no waits between them), and
    the split matvec on the same two streams with a workspace each."""
    monkeypatch.delenv("MX_SYNC_CHECK", raising=False)
    api = require_gpu()
    M, N, K = 512, 1024, 2048                                  # the 8-wave ping-pong kernel, 8 tiles
    say(f"two streams: MXFP8 {M}x{N}x{K}, int4 matvec 8x14336x4096")
    plan = api.mxgemm_create(M, N, K, api.MX_E4M3, api.MX_E4M3)
    sets = [mx_operands(api, api.MX_E4M3, M, N, K, 5100 + 10 * j) for j in range(2)]
    ref = []
    for A, SA, B, SB in sets:                                  # each alone on the default stream
        C = nan_f16((M, N))
        api.mxgemm_run(plan, A, SA, B, SB, C)
        ref.append(bits(C))
    fw, Mv, Kv, Nv = api.MX_INT4, 8, 4096, 14336
    need = api.mxmatvec_workspace_size(Mv, Nv, Kv, fw)
    assert need > 0
    mv = [int_operands(api, fw, Mv, Kv, Nv, 5200 + 10 * j) for j in range(2)]
    wss = [torch.zeros(need, dtype=torch.uint8, device="cuda") for _ in range(2)]
    mref = []
    for (x, W, Ws), ws in zip(mv, wss):
        y = nan_f16((Mv, Nv))
        api.mxmatvec_run(Mv, Nv, Kv, x, W, fw, Ws, y, ws)
        mref.append(bits(y))

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [nan_f16((M, N)) for _ in range(2)]
    ys = [nan_f16((Mv, Nv)) for _ in range(2)]
    torch.cuda.synchronize()
    for rep in range(4):                                       # alternate: both streams stay busy
        for j, s in enumerate(streams):
            with torch.cuda.stream(s):
                api.mxgemm_run(plan, *sets[j], outs[j])
                x, W, Ws = mv[j]
                api.mxmatvec_run(Mv, Nv, Kv, x, W, fw, Ws, ys[j], wss[j])
    torch.cuda.synchronize()
    for j in range(2):
        assert np.array_equal(bits(outs[j]), ref[j]), f"GEMM on stream {j} differs from the call alone"
        assert np.array_equal(bits(ys[j]), mref[j]), f"matvec on stream {j} differs from the call alone"
    plan.close()


def test_graph_capture_replays_match_eager(monkeypatch):
    """An MXFP8 GEMM, an fp16 GEMM, the split matvec with a workspace, the small-M GEMM's block runs
    with a workspace and mxmatvec_run_noalloc, captured in one graph and replayed three times, with
    eager calls on the same workspaces and scratch array between the replays: every replay equals
    the eager result bit for bit."""
    monkeypatch.delenv("MX_SYNC_CHECK", raising=False)
    api = require_gpu()
    M, N, K = 512, 1024, 2048
    say(f"graph: MXFP8 and fp16 {M}x{N}x{K}, int8 matvec 1x14336x4096, int4 block runs 160x12288x1024, "
        f"noalloc int4 8x4096x4096")
    p8 = api.mxgemm_create(M, N, K, api.MX_E4M3, api.MX_E4M3)
    ops8 = mx_operands(api, api.MX_E4M3, M, N, K, 5300)
    p16 = api.mxgemm_create(M, N, K, api.MX_F16, api.MX_F16)
    A16 = dev(synth.uniform_pm1((M, K), 5310).astype(np.float16))
    B16 = dev(synth.uniform_pm1((K, N), 5311).astype(np.float16))
    x1, W1, Ws1 = int_operands(api, api.MX_INT8, 1, 4096, 14336, 5320)
    ws = torch.zeros(api.mxmatvec_workspace_size(1, 14336, 4096, api.MX_INT8), dtype=torch.uint8, device="cuda")
    x8, W8, Ws8 = int_operands(api, api.MX_INT4, 8, 4096, 4096, 5330)
    xr, Wr, Wsr = int_operands(api, api.MX_INT4, 160, 1024, 12288, 5340)
    wsr = torch.zeros(api.mxmatvec_workspace_size(160, 12288, 1024, api.MX_INT4), dtype=torch.uint8, device="cuda")
    assert wsr.numel() > 0                                     # 288 tiles of 64 x 128: block runs

    def run_all(c8, c16, y1, y8, yr):
        api.mxgemm_run(p8, *ops8, c8)
        api.mxgemm_run(p16, A16, None, B16, None, c16)
        api.mxmatvec_run(1, 14336, 4096, x1, W1, api.MX_INT8, Ws1, y1, ws)
        api.mxmatvec_run_noalloc(8, 4096, 4096, x8, W8, api.MX_INT4, Ws8, y8)
        api.mxmatvec_run(160, 12288, 1024, xr, Wr, api.MX_INT4, Wsr, yr, wsr)

    eager = [nan_f16((M, N)), nan_f16((M, N)), nan_f16((1, 14336)), nan_f16((8, 4096)), nan_f16((160, 12288))]
    run_all(*eager)                                            # also the first no-alloc call (set-up)
    want = [bits(t) for t in eager]
    for t in want:
        assert not np.isnan(t.view(np.float16)).any()

    outs = [nan_f16((M, N)), nan_f16((M, N)), nan_f16((1, 14336)), nan_f16((8, 4096)), nan_f16((160, 12288))]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all(*outs)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        again = [nan_f16(t.shape) for t in eager]               # eager work on the same buffers
        run_all(*again)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, w) in enumerate(zip(outs, want)):
            assert np.array_equal(bits(t), w), f"replay {rep}: output {i} differs from the eager call"
        for i, (t, w) in enumerate(zip(again, want)):
            assert np.array_equal(bits(t), w), f"eager call between replays {rep}: output {i} differs"
    p8.close()
    p16.close()
