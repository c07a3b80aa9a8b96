"""The MX_SYNC_CHECK debug switch: with it set, every GPU entry point waits for its stream before it
returns; results and statuses must be those of the same calls without it (no fault is provoked:
the switch only changes when a call returns)."""
import numpy as np
import pytest
import torch

from block_scaled_quantized_amd import synth

from gpu_common import dev, host, nan_f16, require_gpu, say

pytestmark = pytest.mark.gpu


def run_all(api):
    """One call of each GPU entry point on small seeded inputs; returns their outputs on the host."""
    M, N, K = 96, 260, 1024
    a = synth.normal((M, K), 1.0, 3100)
    b = synth.normal((N, K), 0.02, 3101)
    A = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    SA = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
    B = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    SB = torch.empty((N, K // 32), dtype=torch.uint8, device="cuda")
    api.mx_pack_run(api.MX_E4M3, dev(a), M, K, A, SA)
    api.mx_pack_run(api.MX_E4M3, dev(b), N, K, B, SB)
    out = torch.empty((M, K), dtype=torch.float32, device="cuda")
    api.mx_unpack_run(api.MX_E4M3, A, SA, M, K, out)
    plan = api.mxgemm_create(M, N, K, api.MX_E4M3, api.MX_E4M3)
    C = nan_f16((M, N))
    api.mxgemm_run(plan, A, SA, B, SB, C)
    plan.close()
    Kv, Nv = 1024, 512
    w = synth.normal((Kv, Nv), 0.02, 3102)
    x = synth.normal((8, Kv), 1.0, 3103).astype(np.float16)
    W = torch.empty((Kv, Nv), dtype=torch.uint8, device="cuda")
    Ws = torch.empty((Kv // 32, Nv), dtype=torch.float16, device="cuda")
    api.mx_pack_run(api.MX_INT8, dev(w), Kv, Nv, W, Ws)
    y1 = nan_f16((8, Nv))
    need = api.mxmatvec_workspace_size(8, Nv, Kv, api.MX_INT8)
    ws = torch.zeros(max(16, need), dtype=torch.uint8, device="cuda")
    api.mxmatvec_run(8, Nv, Kv, dev(x), W, api.MX_INT8, Ws, y1, ws)
    y2 = nan_f16((8, Nv))
    api.mxmatvec_run_noalloc(8, Nv, Kv, dev(x), W, api.MX_INT8, Ws, y2)
    return [host(t) for t in (A, SA, B, SB, out, C, W, Ws, y1, y2)]


def test_sync_check_same_results(monkeypatch):
    api = require_gpu()
    say("MX_SYNC_CHECK off, then on")
    monkeypatch.delenv("MX_SYNC_CHECK", raising=False)
    ref = run_all(api)
    monkeypatch.setenv("MX_SYNC_CHECK", "1")
    got = run_all(api)
    for r, g in zip(ref, got):
        assert r.dtype == g.dtype and r.shape == g.shape
        assert np.array_equal(r.view(np.uint8), g.view(np.uint8))
    assert not np.isnan(got[5].astype(np.float32)).any() and not np.isnan(got[8].astype(np.float32)).any()
