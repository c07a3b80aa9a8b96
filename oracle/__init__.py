"""CPU oracle for the block-scaled quantized matmul -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package. The product library never does, and this package imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, closed-form decoders, brute-force element
encoder); this module builds it with gcc, loads it with ctypes and wraps each entry point for
numpy arrays. It also holds the acceptance bound used to compare a GPU result with the oracle:

    |C_gpu - C_ref| <= 2^-10 * |C_ref| + 1e-3 * sqrt(K) * R,
    R = sqrt( (1/(M*K*N)) * sum_k (sum_m a_mk^2) (sum_n b_kn^2) )

where a and b are the dequantised operands, i.e. R is the rms of |a_mk * b_kn| over every
(m, k, n) triple. NaN positions must coincide.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

E4M3, E5M2, E2M3, E3M2, E2M1, F16, INT8, INT4 = 0, 1, 2, 3, 4, 16, 32, 33

_lib = None


def build() -> str:
    """Compile oracle.c with gcc (IEEE semantics: no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    L = ctypes.CDLL(_LIB)
    d, u, i, i64, p = ctypes.c_double, ctypes.c_uint, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
    sig = {
        "orc_num_threads": (i, []), "orc_set_threads": (None, [i]),
        "orc_dec_e4m3": (d, [u]), "orc_dec_e5m2": (d, [u]), "orc_dec_e2m1": (d, [u]), "orc_dec_e8m0": (d, [u]),
        "orc_dec_e2m3": (d, [u]), "orc_dec_e3m2": (d, [u]),
        "orc_dec_int4": (d, [u]), "orc_dec_f16": (d, [u]),
        "orc_mx_dot": (d, [i, i, i64, p, p, p, p, i64, i64]),
        "orc_mxgemm_rows": (None, [i, i, i64, i64, i64, p, p, p, p, i64, i64, p]),
        "orc_mxgemm_points": (None, [i, i, i64, p, p, p, p, p, p, i64, p]),
        "orc_f16_dot": (d, [i64, i64, p, p, i64, i64]),
        "orc_gemm_f16_rows": (None, [i64, i64, i64, p, p, i64, i64, p]),
        "orc_gemm_f16_points": (None, [i64, i64, p, p, p, p, i64, p]),
        "orc_matvec_elem": (d, [i, i64, i64, p, p, p, i64, i64]),
        "orc_matvec": (None, [i, i64, i64, i64, p, p, p, p]),
        "orc_dequant": (None, [i, i64, i64, p, p, p]),
        "orc_enc_elem": (u, [i, d]), "orc_floor_log2": (i, [d]),
        "orc_mx_scale_code": (u, [i, d]),
        "orc_mx_quantize": (None, [i, i64, i64, p, p, p]),
        "orc_enc_f16": (u, [d]),
        "orc_int_quantize": (None, [i, i64, i64, p, p, p]),
        "orc_pack_int4": (None, [i64, p, p]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return lib().orc_num_threads()


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


# ---- decoders (vectorised over a code array) -------------------------------------------------

def dec_e4m3(codes) -> np.ndarray:
    return np.array([lib().orc_dec_e4m3(int(c)) for c in np.ravel(codes)]).reshape(np.shape(codes))


def dec_e5m2(codes) -> np.ndarray:
    return np.array([lib().orc_dec_e5m2(int(c)) for c in np.ravel(codes)]).reshape(np.shape(codes))


def dec_e2m3(codes) -> np.ndarray:
    return np.array([lib().orc_dec_e2m3(int(c)) for c in np.ravel(codes)]).reshape(np.shape(codes))


def dec_e3m2(codes) -> np.ndarray:
    return np.array([lib().orc_dec_e3m2(int(c)) for c in np.ravel(codes)]).reshape(np.shape(codes))


def dec_e2m1(codes) -> np.ndarray:
    return np.array([lib().orc_dec_e2m1(int(c)) for c in np.ravel(codes)]).reshape(np.shape(codes))


def dec_e8m0(codes) -> np.ndarray:
    return np.array([lib().orc_dec_e8m0(int(c)) for c in np.ravel(codes)]).reshape(np.shape(codes))


def dec_int4(codes) -> np.ndarray:
    return np.array([lib().orc_dec_int4(int(c)) for c in np.ravel(codes)]).reshape(np.shape(codes))


def dec_f16(bits) -> np.ndarray:
    return np.array([lib().orc_dec_f16(int(c)) for c in np.ravel(bits)]).reshape(np.shape(bits))


# ---- GEMMs -----------------------------------------------------------------------------------

def _mx_shapes(fmt, rows, K):
    if fmt == E2M1:
        return (rows, K // 2)
    return (rows, K // 4 * 3) if fmt in (E2M3, E3M2) else (rows, K)


def mxgemm(fa, fb, A, SA, B, SB, M, N, K, row0=0, nrows=None) -> np.ndarray:
    """fp64 C rows [row0, row0+nrows) of the MX GEMM. B is given K-contiguous ([N][K] codes)."""
    nrows = M - row0 if nrows is None else nrows
    A, SA, B, SB = (np.ascontiguousarray(x, dtype=np.uint8) for x in (A, SA, B, SB))
    assert A.shape == _mx_shapes(fa, M, K) and B.shape == _mx_shapes(fb, N, K)
    assert SA.shape == (M, K // 32) and SB.shape == (N, K // 32)
    C = np.empty((nrows, N), dtype=np.float64)
    lib().orc_mxgemm_rows(fa, fb, M, N, K, _ptr(A), _ptr(SA), _ptr(B), _ptr(SB), row0, nrows, _ptr(C))
    return C


def mxgemm_points(fa, fb, A, SA, B, SB, K, ms, ns) -> np.ndarray:
    A, SA, B, SB = (np.ascontiguousarray(x, dtype=np.uint8) for x in (A, SA, B, SB))
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    out = np.empty(ms.shape[0], dtype=np.float64)
    lib().orc_mxgemm_points(fa, fb, K, _ptr(A), _ptr(SA), _ptr(B), _ptr(SB), _ptr(ms), _ptr(ns),
                            ms.shape[0], _ptr(out))
    return out


def relu(C) -> np.ndarray:
    """Epilogue ReLU of the "Running inline ML operations in a shader with Metal 4" sample, section
    "Combine an element-wise function": every negative element of the product becomes zero, the
    sample writing it as max(value, 0). max is taken with IEEE maxNum semantics, so a NaN element
    becomes 0 (the reading of max for a NaN argument). Applied to the fp64 product; rounding to
    fp16 afterwards gives the same values, since nearest-even rounding keeps the sign and zero."""
    return np.fmax(np.asarray(C, dtype=np.float64), 0.0)


def gemm_f16(A16, B16, row0=0, nrows=None) -> np.ndarray:
    """fp64 C = A @ B for binary16 A [M][K], B [K][N] (numpy float16 arrays)."""
    A = np.ascontiguousarray(A16, dtype=np.float16).view(np.uint16)
    B = np.ascontiguousarray(B16, dtype=np.float16).view(np.uint16)
    M, K = A.shape
    N = B.shape[1]
    nrows = M - row0 if nrows is None else nrows
    C = np.empty((nrows, N), dtype=np.float64)
    lib().orc_gemm_f16_rows(M, N, K, _ptr(A), _ptr(B), row0, nrows, _ptr(C))
    return C


def gemm_f16_points(A16, B16, ms, ns) -> np.ndarray:
    A = np.ascontiguousarray(A16, dtype=np.float16).view(np.uint16)
    B = np.ascontiguousarray(B16, dtype=np.float16).view(np.uint16)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    out = np.empty(ms.shape[0], dtype=np.float64)
    lib().orc_gemm_f16_points(B.shape[1], A.shape[1], _ptr(A), _ptr(B), _ptr(ms), _ptr(ns), ms.shape[0], _ptr(out))
    return out


def matvec(fw, x16, W, Ws16, K, N) -> np.ndarray:
    """fp64 y [M][N] of the block-scaled dequant matvec. W is int8 [K][N] or packed int4 bytes."""
    x = np.ascontiguousarray(x16, dtype=np.float16).view(np.uint16)
    Wb = np.ascontiguousarray(W).view(np.uint8)
    Ws = np.ascontiguousarray(Ws16, dtype=np.float16).view(np.uint16)
    M = x.shape[0]
    assert x.shape == (M, K) and Ws.shape == (K // 32, N)
    assert Wb.size == (K * N if fw == INT8 else K * N // 2)
    y = np.empty((M, N), dtype=np.float64)
    lib().orc_matvec(fw, M, N, K, _ptr(x), _ptr(Wb), _ptr(Ws), _ptr(y))
    return y


def matvec_elem(fw, x16, W, Ws16, K, N, m, n) -> float:
    x = np.ascontiguousarray(x16, dtype=np.float16).view(np.uint16)
    Wb = np.ascontiguousarray(W).view(np.uint8)
    Ws = np.ascontiguousarray(Ws16, dtype=np.float16).view(np.uint16)
    return lib().orc_matvec_elem(fw, N, K, _ptr(x), _ptr(Wb), _ptr(Ws), m, n)


def dequant(fmt, codes, scales, rows, cols) -> np.ndarray:
    codes = np.ascontiguousarray(codes).view(np.uint8)
    scales = np.ascontiguousarray(scales)
    if fmt in (INT8, INT4):
        scales = scales.astype(np.float16).view(np.uint16)
    out = np.empty((rows, cols), dtype=np.float32)
    lib().orc_dequant(fmt, rows, cols, _ptr(codes), _ptr(scales), _ptr(out))
    return out


# ---- encoders --------------------------------------------------------------------------------

def enc_elem(fmt, v) -> np.ndarray:
    return np.array([lib().orc_enc_elem(fmt, float(x)) for x in np.ravel(v)], dtype=np.uint8).reshape(np.shape(v))


def floor_log2(a: float) -> int:
    return lib().orc_floor_log2(float(a))


def mx_scale_code(fmt, amax: float) -> int:
    return lib().orc_mx_scale_code(fmt, float(amax))


def mx_quantize(fmt, src):
    """Quantise fp32 [rows][cols] in 32-wide blocks along cols -> (codes, e8m0 scales)."""
    src = np.ascontiguousarray(src, dtype=np.float32)
    rows, cols = src.shape
    codes = np.zeros(_mx_shapes(fmt, rows, cols), dtype=np.uint8)
    scales = np.zeros((rows, cols // 32), dtype=np.uint8)
    lib().orc_mx_quantize(fmt, rows, cols, _ptr(src), _ptr(codes), _ptr(scales))
    return codes, scales


def enc_f16(x: float) -> int:
    return lib().orc_enc_f16(float(x))


def int_quantize(fw, w):
    """Symmetric per-32-row quantisation of W [K][N] fp32 -> (q int8 [K][N], fp16 scales [K/32][N]).

    For int4 the returned q is the unpacked nibble value (-7..7); see pack_int4."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    K, N = w.shape
    q = np.zeros((K, N), dtype=np.int8)
    s = np.zeros((K // 32, N), dtype=np.uint16)
    lib().orc_int_quantize(127 if fw == INT8 else 7, K, N, _ptr(w), _ptr(q), _ptr(s))
    return q, s.view(np.float16)


def pack_int4(q) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    out = np.zeros(q.size // 2, dtype=np.uint8)
    lib().orc_pack_int4(q.size, _ptr(q), _ptr(out))
    return out.reshape(q.shape[0], q.shape[1] // 2)


# ---- acceptance bound ------------------------------------------------------------------------

def rms_ab(a_deq: np.ndarray, b_deq_kn: np.ndarray) -> float:
    """R = rms of |a_mk b_kn| over all (m,k,n): sqrt(sum_k (sum_m a^2)(sum_n b^2) / (M K N))."""
    a = np.asarray(a_deq, dtype=np.float64)
    b = np.asarray(b_deq_kn, dtype=np.float64)
    M, K = a.shape
    N = b.shape[1]
    ra = np.sum(a * a, axis=0)
    rb = np.sum(b * b, axis=1)
    return float(np.sqrt(np.sum(ra * rb) / (M * K * N)))


def bound(c_ref: np.ndarray, K: int, R: float) -> np.ndarray:
    return 2.0 ** -10 * np.abs(c_ref) + 1e-3 * np.sqrt(K) * R


F16_OVERFLOW = 65520.0   # binary16 round-to-nearest-even sends |x| >= 65520 to Inf


def check(c_gpu, c_ref, K, R):
    """Return (ok, worst err/bound, number of violations). NaN positions must coincide.

    The output is binary16 rounded to nearest even, so an infinite GPU output is correct exactly
    when the reference, moved by at most its bound toward larger magnitude, reaches the fp16
    overflow threshold with the same sign; such outputs count as err/bound = 0. An infinite
    reference (an infinite operand, E5M2's Inf codes) is met only by the same infinity: its bound
    is infinite too, so it is compared for equality instead."""
    c_gpu = np.asarray(c_gpu, dtype=np.float64)
    c_ref = np.asarray(c_ref, dtype=np.float64)
    nan_ok = np.array_equal(np.isnan(c_gpu), np.isnan(c_ref))
    fin = ~np.isnan(c_ref) & ~np.isnan(c_gpu)
    g, r = c_gpu[fin], c_ref[fin]
    with np.errstate(invalid="ignore"):
        bnd = bound(r, K, R)
        rinf = np.isinf(r)
        inf = np.isinf(g) & ~rinf
        inf_ok = inf & (np.sign(g) == np.sign(r)) & (np.abs(r) + bnd >= F16_OVERFLOW)
        err = np.where(inf | rinf, 0.0, np.abs(g - r))
        ok_each = np.where(rinf, g == r, np.where(inf, inf_ok, err <= bnd))
        ratio_each = np.where(rinf, np.where(g == r, 0.0, np.inf),
                              np.where(inf, np.where(inf_ok, 0.0, np.inf), err / bnd))
    ratio = float(np.max(ratio_each)) if g.size else 0.0
    bad = int(np.sum(~ok_each))
    return (nan_ok and bad == 0), ratio, bad
