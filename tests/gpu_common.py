"""Helpers shared by the GPU parity tests: device allocation through torch and calls through the
C ABI (block_scaled_quantized_amd.api). No arithmetic of the method lives here."""
import sys

import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X (gfx950) device; select them with -m gpu")
    from block_scaled_quantized_amd import api
    return api


def say(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def empty(shape, dtype) -> torch.Tensor:
    return torch.empty(shape, dtype=dtype, device="cuda")


def gpu_mx_pack(api, fmt, src: np.ndarray):
    rows, cols = src.shape
    cs, ss = api.mx_shapes(fmt, rows, cols)
    codes = empty(cs, torch.uint8)
    scales = empty(ss, torch.uint8)
    api.mx_pack_run(fmt, dev(src.astype(np.float32)), rows, cols, codes, scales)
    return codes, scales


def gpu_int_pack(api, fw, w: np.ndarray):
    K, N = w.shape
    cs, ss = api.int_shapes(fw, K, N)
    codes = empty(cs, torch.uint8)
    scales = empty(ss, torch.float16)
    api.mx_pack_run(fw, dev(w.astype(np.float32)), K, N, codes, scales)
    return codes, scales


def gpu_gemm(api, fa, A, SA, B, SB, M, N, K, flags=0, fb=None) -> np.ndarray:
    plan = api.mxgemm_create(M, N, K, fa, fa if fb is None else fb, flags)
    C = empty((M, N), torch.float16)
    api.mxgemm_run(plan, A, SA, B, SB, C)
    out = host(C).astype(np.float64)
    plan.close()
    return out


def bitequal_f32(a: np.ndarray, b: np.ndarray) -> bool:
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    if not np.array_equal(np.isnan(a), np.isnan(b)):
        return False
    f = ~np.isnan(a)
    return np.array_equal(a.view(np.uint32)[f], b.view(np.uint32)[f])
