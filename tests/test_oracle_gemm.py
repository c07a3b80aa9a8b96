"""Pins of the oracle's GEMM, matvec and dequant against what the mathematics fixes.

- Unit scales reduce the MX GEMM to a plain fp8 matmul: compared bit-for-bit with torch's fp64
  matmul of torch-decoded E4M3 / E5M2 (all partial sums are exact in fp64 at these sizes).
- Tiny shapes with random scales: the exact rational sum (fractions.Fraction) within the fp64
  recursive-summation bound.
- Scale shift and block locality invariants, on data chosen so every sum is exact.
- NaN scale / NaN code propagation.
- fp16 GEMM and matvec against numpy/torch fp64 products within the summation bound.
- Dequant against torch fp32 products (exact products rounded once).
- The acceptance bound has teeth: plausible mistakes fail it, fp16 rounding of the truth passes.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from block_scaled_quantized_amd import synth
from conftest import read_golden

E4M3_NAN = (0x7F, 0xFF)


def e2m1_table():
    return np.array([float(v) for _, v in read_golden("e2m1_values.txt")])


def torch_e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64)


def unpack_nibbles_k(codes_packed):
    """[rows][K/2] bytes -> [rows][K] nibbles, even k in the low nibble (numpy bit ops)."""
    lo = codes_packed & 0xF
    hi = codes_packed >> 4
    out = np.empty((codes_packed.shape[0], codes_packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def sum_bound(terms_abs_sum, n):
    return n * 2.0 ** -53 * terms_abs_sum * 1.01


@pytest.mark.parametrize("M,N,K", [(7, 5, 32), (16, 16, 128), (33, 17, 256)])
def test_mx_e4m3_unit_scales_is_plain_fp8_matmul(orc, M, N, K):
    A = synth.random_bytes((M, K), 11, exclude=E4M3_NAN)
    B = synth.random_bytes((N, K), 12, exclude=E4M3_NAN)
    SA = np.full((M, K // 32), 127, np.uint8)
    SB = np.full((N, K // 32), 127, np.uint8)
    C = orc.mxgemm(orc.E4M3, orc.E4M3, A, SA, B, SB, M, N, K)
    ref = (torch_e4m3(A) @ torch_e4m3(B).T).numpy()
    assert np.array_equal(C, ref)


E5M2_NONFINITE = tuple(c for c in range(256) if (c & 0x7C) == 0x7C)   # Inf and NaN codes


def torch_e5m2(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e5m2).to(torch.float64)


@pytest.mark.parametrize("M,N,K", [(7, 5, 32), (16, 16, 128)])
def test_mx_e5m2_unit_scales_is_plain_fp8_matmul(orc, M, N, K):
    """E5M2, and E5M2 x E4M3, at unit scales: torch's fp64 matmul of torch-decoded codes. Exponent
    fields 8..23 (values 2^-7 .. 1.75*2^8, zero included) keep every product a multiple of 2^-16
    below 2^18, so all partial sums are exact in fp64 whatever the order."""
    g = np.random.Generator(np.random.PCG64(15 + K))

    def codes(shape):
        e = g.integers(8, 24, size=shape)
        e[g.random(shape) < 0.05] = 0                        # some zeros and subnormal-field codes
        return ((g.integers(0, 2, size=shape) << 7) | (e << 2) | g.integers(0, 4, size=shape)).astype(np.uint8)
    A = codes((M, K))
    B = codes((N, K))
    SA = np.full((M, K // 32), 127, np.uint8)
    SB = np.full((N, K // 32), 127, np.uint8)
    C = orc.mxgemm(orc.E5M2, orc.E5M2, A, SA, B, SB, M, N, K)
    assert np.array_equal(C, (torch_e5m2(A) @ torch_e5m2(B).T).numpy())
    B8 = synth.random_bytes((N, K), 18 + K, exclude=E4M3_NAN)
    C = orc.mxgemm(orc.E5M2, orc.E4M3, A, SA, B8, SB, M, N, K)
    assert np.array_equal(C, (torch_e5m2(A) @ torch_e4m3(B8).T).numpy())


@pytest.mark.parametrize("fa,fb", [(2, 2), (3, 3), (2, 3)])
def test_mx_fp6_unit_scales_is_plain_matmul(orc, fa, fb):
    """FP6 at unit scales: numpy's matmul of the decoded elements (multiples of 2^-4 below 28, so
    every sum is exact), with the 6-bit fields unpacked by numpy's little-endian bit stream."""
    M, N, K = 9, 11, 128
    g = np.random.Generator(np.random.PCG64(40 + fa + fb))
    def pack(codes):
        bits = ((codes[..., None] >> np.arange(6)) & 1).astype(np.uint8).reshape(codes.shape[0], -1)
        return np.packbits(bits, axis=1, bitorder="little")
    ca, cb = g.integers(0, 64, (M, K)), g.integers(0, 64, (N, K))
    names = {2: "e2m3", 3: "e3m2"}
    a = getattr(orc, "dec_" + names[fa])(ca)
    b = getattr(orc, "dec_" + names[fb])(cb)
    SA = np.full((M, K // 32), 127, np.uint8)
    SB = np.full((N, K // 32), 127, np.uint8)
    C = orc.mxgemm(fa, fb, pack(ca), SA, pack(cb), SB, M, N, K)
    assert np.array_equal(C, a @ b.T)


def test_mx_e2m1_unit_scales_is_plain_fp4_matmul(orc):
    M, N, K = 9, 11, 96
    A = synth.random_bytes((M, K // 2), 13)
    B = synth.random_bytes((N, K // 2), 14)
    SA = np.full((M, K // 32), 127, np.uint8)
    SB = np.full((N, K // 32), 127, np.uint8)
    tab = e2m1_table()
    a = tab[unpack_nibbles_k(A)]
    b = tab[unpack_nibbles_k(B)]
    C = orc.mxgemm(orc.E2M1, orc.E2M1, A, SA, B, SB, M, N, K)
    assert np.array_equal(C, a @ b.T)   # multiples of 1/4, |sum| < 2^12: exact in any order


@pytest.mark.parametrize("fmt", [0, 4])
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (2, 3, 64), (4, 4, 96), (3, 1, 96)])
def test_mx_tiny_brute_force_fraction(orc, fmt, M, N, K):
    seed = 100 + M * 7 + N * 3 + K + fmt
    if fmt == 0:
        A = synth.random_bytes((M, K), seed, exclude=E4M3_NAN)
        B = synth.random_bytes((N, K), seed + 1, exclude=E4M3_NAN)
        val = lambda c: Fraction(float(torch_e4m3(np.array([c], np.uint8))[0]))
        elem = lambda row, k: row[k]
    else:
        A = synth.random_bytes((M, K // 2), seed)
        B = synth.random_bytes((N, K // 2), seed + 1)
        tab = e2m1_table()
        val = lambda c: Fraction(tab[c])
        elem = lambda row, k: (row[k // 2] >> (4 * (k % 2))) & 0xF
    SA = synth.random_ints((M, K // 32), 117, 137, seed + 2)
    SB = synth.random_ints((N, K // 32), 117, 137, seed + 3)
    C = orc.mxgemm(fmt, fmt, A, SA, B, SB, M, N, K)
    for m in range(M):
        for n in range(N):
            exact = Fraction(0)
            absum = Fraction(0)
            for k in range(K):
                t = val(elem(A[m], k)) * Fraction(2) ** (int(SA[m, k // 32]) - 127) \
                    * val(elem(B[n], k)) * Fraction(2) ** (int(SB[n, k // 32]) - 127)
                exact += t
                absum += abs(t)
            assert abs(Fraction(C[m, n]) - exact) <= Fraction(sum_bound(float(absum), K))


def _exact_e4m3_codes(shape, seed):
    # Normal codes with exponent field 4..10 (values 2^-3 .. 1.875*2^3): with scale codes in
    # [124, 130] every product is a multiple of 2^-18 below 2^14, so all sums up to K=256 are exact.
    g = np.random.Generator(np.random.PCG64(seed))
    e = g.integers(4, 11, size=shape)
    f = g.integers(0, 8, size=shape)
    s = g.integers(0, 2, size=shape)
    return ((s << 7) | (e << 3) | f).astype(np.uint8)


def test_mx_scale_shift_invariant(orc):
    M, N, K = 6, 5, 256
    A = _exact_e4m3_codes((M, K), 21)
    B = _exact_e4m3_codes((N, K), 22)
    SA = synth.random_ints((M, K // 32), 124, 130, 23)
    SB = synth.random_ints((N, K // 32), 124, 130, 24)
    C = orc.mxgemm(0, 0, A, SA, B, SB, M, N, K)
    # single-block partials: zero every code outside block b
    parts = []
    for b in range(K // 32):
        Ab = np.zeros_like(A)
        Ab[:, 32 * b:32 * b + 32] = A[:, 32 * b:32 * b + 32]
        parts.append(orc.mxgemm(0, 0, Ab, SA, B, SB, M, N, K))
    assert np.array_equal(sum(parts), C)                     # block locality: blocks add up
    m, b, d = 3, 5, 2
    SA2 = SA.copy()
    SA2[m, b] += d
    C2 = orc.mxgemm(0, 0, A, SA2, B, SB, M, N, K)
    expect = C.copy()
    expect[m] += (2 ** d - 1) * parts[b][m]
    assert np.array_equal(C2, expect)                        # only row m moves, by (2^d-1)*partial
    n = 2
    SB2 = SB.copy()
    SB2[n, b] -= 1
    C3 = orc.mxgemm(0, 0, A, SA, B, SB2, M, N, K)
    expect = C.copy()
    expect[:, n] -= 0.5 * parts[b][:, n]
    assert np.array_equal(C3, expect)                        # only column n moves


def test_mx_points_equal_rows_and_transpose(orc):
    M, N, K = 12, 9, 128
    A = synth.random_bytes((M, K), 31, exclude=E4M3_NAN)
    B = synth.random_bytes((N, K), 32, exclude=E4M3_NAN)
    SA = synth.random_ints((M, K // 32), 120, 134, 33)
    SB = synth.random_ints((N, K // 32), 120, 134, 34)
    C = orc.mxgemm(0, 0, A, SA, B, SB, M, N, K)
    ms, ns = synth.sample_points(M, N, 40, 35)
    assert np.array_equal(orc.mxgemm_points(0, 0, A, SA, B, SB, K, ms, ns), C[ms, ns])
    assert np.array_equal(orc.mxgemm(0, 0, A, SA, B, SB, M, N, K, row0=4, nrows=3), C[4:7])
    Ct = orc.mxgemm(0, 0, B, SB, A, SA, N, M, K)             # swapping operands transposes C
    assert np.array_equal(Ct, C.T)


def test_mx_nan_propagation(orc):
    M, N, K = 4, 4, 64
    A = synth.random_bytes((M, K), 41, exclude=E4M3_NAN)
    B = synth.random_bytes((N, K), 42, exclude=E4M3_NAN)
    SA = np.full((M, K // 32), 127, np.uint8)
    SB = np.full((N, K // 32), 127, np.uint8)
    SA[1, 1] = 0xFF                 # NaN scale: all of row 1
    B2 = B.copy()
    B2[2, 5] = 0x7F                 # NaN code: all of column 2
    C = orc.mxgemm(0, 0, A, SA, B2, SB, M, N, K)
    nan = np.isnan(C)
    assert nan[1].all() and nan[:, 2].all()
    assert nan.sum() == M + N - 1


def test_f16_gemm_vs_torch(orc):
    M, N, K = 24, 20, 200
    A = synth.uniform_pm1((M, K), 51).astype(np.float16)
    B = synth.uniform_pm1((K, N), 52).astype(np.float16)
    C = orc.gemm_f16(A, B)
    ref = (torch.from_numpy(A).double() @ torch.from_numpy(B).double()).numpy()
    absum = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
    assert np.all(np.abs(C - ref) <= 2 * sum_bound(absum, K))
    # integer-valued inputs: exact in any order
    Ai = synth.random_ints((M, K), 0, 16, 53).astype(np.float16) - np.float16(8)
    Bi = synth.random_ints((K, N), 0, 16, 54).astype(np.float16) - np.float16(8)
    assert np.array_equal(orc.gemm_f16(Ai, Bi), Ai.astype(np.float64) @ Bi.astype(np.float64))
    ms, ns = synth.sample_points(M, N, 30, 55)
    assert np.array_equal(orc.gemm_f16_points(A, B, ms, ns), C[ms, ns])


@pytest.mark.parametrize("fw", [32, 33])
def test_matvec_vs_numpy_dequant_then_dot(orc, fw):
    M, K, N = 3, 128, 48
    x = synth.normal((M, K), 1.0, 61).astype(np.float16)
    if fw == 32:
        q = synth.random_bytes((K, N), 62).view(np.int8)
        W = q
    else:
        W = synth.random_bytes((K, N // 2), 62)
        q = np.empty((K, N), np.int8)
        flat = W.reshape(-1)
        qf = q.reshape(-1)
        qf[0::2] = ((flat.astype(np.int8) << 4).astype(np.int8) >> 4)
        qf[1::2] = (flat.astype(np.int8) >> 4)
    s = (synth.normal((K // 32, N), 0.01, 63)).astype(np.float16)
    y = orc.matvec(fw, x, W, s, K, N)
    wdeq = q.astype(np.float64) * np.repeat(s.astype(np.float64), 32, axis=0)
    ref = x.astype(np.float64) @ wdeq
    absum = np.abs(x.astype(np.float64)) @ np.abs(wdeq)
    assert np.all(np.abs(y - ref) <= 2 * sum_bound(absum, K))
    assert orc.matvec_elem(fw, x, W, s, K, N, 2, 7) == y[2, 7]


def test_dequant_mx_vs_torch(orc):
    rows, cols = 8, 128
    A = synth.random_bytes((rows, cols), 71)
    S = synth.random_bytes((rows, cols // 32), 72)
    S[0, 0], S[1, 1], S[2, 2] = 0, 254, 255          # smallest, largest (overflow), NaN
    out = orc.dequant(0, A, S, rows, cols)
    a = torch.from_numpy(A).view(torch.float8_e4m3fn).float()
    s = torch.from_numpy(np.repeat(S, 32, axis=1)).view(torch.float8_e8m0fnu).float()
    ref = (a * s).numpy()
    assert np.array_equal(out.view(np.uint32)[~np.isnan(ref)], ref.view(np.uint32)[~np.isnan(ref)])
    assert np.array_equal(np.isnan(out), np.isnan(ref))
    # E5M2: every code (Inf and NaN included) times scale, fp32 product
    out5 = orc.dequant(1, A, S, rows, cols)
    ref5 = (torch.from_numpy(A).view(torch.float8_e5m2).float() * s).numpy()
    fin5 = ~np.isnan(ref5)
    assert np.array_equal(out5.view(np.uint32)[fin5], ref5.view(np.uint32)[fin5])
    assert np.array_equal(np.isnan(out5), np.isnan(ref5))
    # E2M1: table value times scale, fp32 product
    A4 = synth.random_bytes((rows, cols // 2), 73)
    out4 = orc.dequant(4, A4, S, rows, cols)
    v = torch.from_numpy(e2m1_table()[unpack_nibbles_k(A4)].astype(np.float32))
    ref4 = (v * s).numpy()
    fin = ~np.isnan(ref4)
    assert np.array_equal(out4.view(np.uint32)[fin], ref4.view(np.uint32)[fin])
    assert np.array_equal(np.isnan(out4), np.isnan(ref4))


def test_dequant_int_vs_torch(orc):
    K, N = 64, 16
    q = synth.random_bytes((K, N), 81)
    s = synth.normal((K // 32, N), 0.01, 82).astype(np.float16)
    out = orc.dequant(32, q, s, K, N)
    ref = (torch.from_numpy(q.view(np.int8)).float() * torch.from_numpy(np.repeat(s, 32, 0)).float()).numpy()
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    W4 = synth.random_bytes((K, N // 2), 83)
    out4 = orc.dequant(33, W4, s, K, N)
    flat = W4.reshape(-1)
    qq = np.empty(K * N, np.int8)
    qq[0::2] = ((flat.astype(np.int8) << 4).astype(np.int8) >> 4)
    qq[1::2] = flat.astype(np.int8) >> 4
    ref4 = (torch.from_numpy(qq.reshape(K, N)).float() * torch.from_numpy(np.repeat(s, 32, 0)).float()).numpy()
    assert np.array_equal(out4.view(np.uint32), ref4.view(np.uint32))


def test_bound_has_teeth(orc):
    """Mutations the GPU could plausibly make fail the acceptance bound; fp16 rounding passes."""
    M, N, K = 64, 64, 256
    a_src = synth.normal((M, K), 1.0, 91)
    b_src = synth.normal((N, K), 1.0, 92)
    A, SA = orc.mx_quantize(0, a_src)
    B, SB = orc.mx_quantize(0, b_src)
    C = orc.mxgemm(0, 0, A, SA, B, SB, M, N, K)
    R = orc.rms_ab(orc.dequant(0, A, SA, M, K), orc.dequant(0, B, SB, N, K).T)
    ok, ratio, _ = orc.check(C.astype(np.float16).astype(np.float64), C, K, R)
    assert ok and ratio < 0.6
    SA2 = SA.copy()
    SA2[5, 3] += 1                                   # one scale block off by x2
    ok, _, _ = orc.check(orc.mxgemm(0, 0, A, SA2, B, SB, M, N, K), C, K, R)
    assert not ok
    A3 = A.copy()                                    # two K-blocks swapped in A only
    A3[:, 0:32], A3[:, 32:64] = A[:, 32:64], A[:, 0:32]
    ok, _, _ = orc.check(orc.mxgemm(0, 0, A3, SA, B, SB, M, N, K), C, K, R)
    assert not ok
    A4 = A.copy()                                    # last K-block dropped
    A4[:, K - 32:] = 0
    ok, _, _ = orc.check(orc.mxgemm(0, 0, A4, SA, B, SB, M, N, K), C, K, R)
    assert not ok
    ok, _, _ = orc.check(C.T.copy(), C, K, R)        # transposed output
    assert not ok


def test_relu_special_values(orc):
    """The epilogue ReLU: negatives (and -Inf) to zero, positives and +Inf kept, NaN to zero (IEEE
    maxNum, the reading of the sample's max(value, 0) for a NaN), zero kept as a zero."""
    x = np.array([-1.0, -0.0, 0.0, 2.5, np.nan, -np.inf, np.inf, -1e-300, 65504.0])
    y = orc.relu(x)
    assert y.tolist()[:4] == [0.0, 0.0, 0.0, 2.5]
    assert y[4] == 0.0 and y[5] == 0.0 and y[6] == np.inf and y[7] == 0.0 and y[8] == 65504.0
    C = orc.mxgemm(0, 0, np.full((2, 32), 0x38, np.uint8), np.array([[127], [127]], np.uint8),
                   np.array([[0x38] * 32, [0xB8] * 32], np.uint8), np.array([[127], [127]], np.uint8), 2, 2, 32)
    assert C.tolist() == [[32.0, -32.0], [32.0, -32.0]]          # 32 products of +-1
    assert orc.relu(C).tolist() == [[32.0, 0.0], [32.0, 0.0]]


@pytest.mark.parametrize("M,K,N,seed", [(3, 5, 4, 1), (7, 2, 11, 2), (1, 9, 1, 3), (6, 13, 2, 4)])
def test_rms_ab_is_the_triplewise_rms(orc, M, K, N, seed):
    """R of the acceptance bound is the root mean square of |a_mk b_kn| over every (m, k, n)
    triple: summed here one triple at a time with math.fsum (an exactly rounded sum), on
    non-square shapes with M, K and N all different, so a transposed operand, a sum over the wrong
    axis or a wrong normaliser (M*N, K, ...) fails."""
    import math
    g = np.random.Generator(np.random.PCG64(seed))
    a = g.standard_normal((M, K)) * g.integers(1, 5, size=(M, K))
    b = g.standard_normal((K, N)) * 3.0
    terms = [(a[m, k] * b[k, n]) ** 2 for m in range(M) for k in range(K) for n in range(N)]
    want = math.sqrt(math.fsum(terms) / (M * K * N))
    assert abs(orc.rms_ab(a, b) - want) <= 1e-13 * want
    # a scaled operand scales R by the same factor; a single nonzero triple gives |a b| / sqrt(MKN)
    assert abs(orc.rms_ab(2.0 * a, b) - 2.0 * want) <= 1e-13 * want
    a1 = np.zeros((M, K))
    b1 = np.zeros((K, N))
    a1[M - 1, K - 1], b1[K - 1, N - 1] = 3.0, -5.0
    assert orc.rms_ab(a1, b1) == pytest.approx(15.0 / math.sqrt(M * K * N), rel=1e-15)


def test_check_infinite_reference_needs_the_same_infinity(orc):
    """An infinite reference (E5M2 Inf codes) is met only by the same infinity: a finite or
    opposite output fails even though the bound is infinite there."""
    ref = np.array([np.inf, -np.inf, 1.0])
    assert orc.check(np.array([np.inf, -np.inf, 1.0]), ref, 32, 1.0)[0]
    assert not orc.check(np.array([60000.0, -np.inf, 1.0]), ref, 32, 1.0)[0]
    assert not orc.check(np.array([np.inf, np.inf, 1.0]), ref, 32, 1.0)[0]
    assert not orc.check(np.array([np.nan, -np.inf, 1.0]), ref, 32, 1.0)[0]
