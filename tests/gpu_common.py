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


def nan_f16(shape) -> torch.Tensor:
    """An fp16 output buffer filled with the NaN 0x7E00, so that every output a kernel fails to
    write shows up as NaN, whatever the allocator hands back."""
    return torch.full(shape, float("nan"), dtype=torch.float16, device="cuda")


def sentinel_f32(shape) -> torch.Tensor:
    """An fp32 output buffer filled with 12345.678 (a value no unpack at the tested scales writes)."""
    return torch.full(shape, 12345.678, dtype=torch.float32, device="cuda")


def poisoned_u8(shape) -> torch.Tensor:
    """A code / scale buffer filled with 0x5A before a pack writes it."""
    return torch.full(shape, 0x5A, dtype=torch.uint8, device="cuda")


def gpu_mx_pack(api, fmt, src: np.ndarray):
    rows, cols = src.shape
    cs, ss = api.mx_shapes(fmt, rows, cols)
    codes = poisoned_u8(cs)
    scales = poisoned_u8(ss)
    api.mx_pack_run(fmt, dev(src.astype(np.float32)), rows, cols, codes, scales)
    return codes, scales


def gpu_int_pack(api, fw, w: np.ndarray):
    K, N = w.shape
    cs, ss = api.int_shapes(fw, K, N)
    codes = poisoned_u8(cs)
    scales = torch.full(ss, 3.0, dtype=torch.float16, device="cuda")   # sentinel scale
    api.mx_pack_run(fw, dev(w.astype(np.float32)), K, N, codes, scales)
    return codes, scales


def gpu_gemm(api, fa, A, SA, B, SB, M, N, K, flags=0, fb=None) -> np.ndarray:
    plan = api.mxgemm_create(M, N, K, fa, fa if fb is None else fb, flags)
    C = nan_f16((M, N))
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
