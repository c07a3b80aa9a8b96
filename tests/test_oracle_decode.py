"""Pins of the oracle's decoders against what fixes them independently of the oracle.

E4M3 and E8M0: torch's float8_e4m3fn / float8_e8m0fnu dtypes (an independent library) and the
OCP special values in tests/golden. E2M1: the OCP value table in tests/golden and its embedding
into torch's E4M3. int4: numpy's arithmetic-shift sign extension and the page's packing rule
worked by hand. binary16: numpy's float16.
"""
import math

import numpy as np
import pytest
import torch

from conftest import read_golden


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    f = ~np.isnan(a)
    assert np.array_equal(a[f], b[f])
    assert np.array_equal(np.signbit(a[f]), np.signbit(b[f]))


def test_e4m3_all_codes_match_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    _same(orc.dec_e4m3(codes), ref)


def test_e5m2_all_codes_match_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    _same(orc.dec_e5m2(codes), ref)


@pytest.mark.parametrize("fp6,fp8_dtype,vmax,vmin", [("e2m3", torch.float8_e4m3fn, 7.5, 0.125),
                                                       ("e3m2", torch.float8_e5m2, 28.0, 0.0625)])
def test_fp6_embeds_into_torch_fp8(orc, fp6, fp8_dtype, vmax, vmin):
    """Every FP6 value lies on the fp8 grid with the same mantissa width (E2M3 in E4M3, E3M2 in
    E5M2, both decoded by torch), positive codes 0..31 increase strictly from 0 to the largest
    element, the smallest nonzero is the subnormal unit, each binade holds the same number of
    codes, and bit 5 is the sign."""
    dec = getattr(orc, "dec_" + fp6)
    grid = set(torch.arange(256, dtype=torch.uint8).view(fp8_dtype).to(torch.float64).numpy().tolist())
    pos = dec(np.arange(32))
    neg = dec(np.arange(32, 64))
    assert all(v in grid for v in pos)
    assert np.all(np.diff(pos) > 0) and pos[0] == 0.0 and pos[-1] == vmax and pos[1] == vmin
    assert np.array_equal(neg, -pos) and np.signbit(neg[0])
    per = 8 if fp6 == "e2m3" else 4                     # codes per binade: 2^mantissa bits
    normals = pos[per:]
    expo = np.floor(np.log2(normals))
    assert all(np.sum(expo == e) == per for e in np.unique(expo))


def test_e4m3_golden_specials(orc):
    for code, val in read_golden("e4m3_specials.txt"):
        got = orc.dec_e4m3([int(code, 16)])[0]
        _same([got], [float(val)])


def test_e8m0_all_codes_match_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    _same(orc.dec_e8m0(codes), ref)


def test_e8m0_golden(orc):
    for code, lg in read_golden("e8m0_specials.txt"):
        got = orc.dec_e8m0([int(code, 16)])[0]
        if lg == "nan":
            assert math.isnan(got)
        else:
            assert got == math.ldexp(1.0, int(lg))


def test_e2m1_golden_table(orc):
    rows = read_golden("e2m1_values.txt")
    assert len(rows) == 16
    for code, val in rows:
        _same(orc.dec_e2m1([int(code)]), [float(val)])


def test_e2m1_embeds_into_torch_e4m3(orc):
    # Every E2M1 value is an E4M3 value: exponent field e -> e+6, mantissa bit m -> m<<2 for normal
    # codes; the subnormal 0.5 is E4M3 exponent field 6. Checked through torch's decoder.
    for n in range(16):
        s, e, m = n >> 3, (n >> 1) & 3, n & 1
        if e == 0 and m == 0:
            b = 0
        elif e == 0:
            b = 6 << 3
        else:
            b = ((e + 6) << 3) | (m << 2)
        b |= s << 7
        ref = torch.tensor([b], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).item()
        _same(orc.dec_e2m1([n]), [ref])


def test_int4_nibbles_sign_extension(orc):
    by = np.arange(256, dtype=np.uint8)
    lo = ((by.astype(np.int8) << 4).astype(np.int8) >> 4).astype(np.float64)   # arithmetic shift
    hi = (by.astype(np.int8) >> 4).astype(np.float64)
    assert np.array_equal(orc.dec_int4(by & 0xF), lo)
    assert np.array_equal(orc.dec_int4(by >> 4), hi)


def test_int4_pack_golden(orc):
    for v0, v1, byte in read_golden("int4_pack_examples.txt"):
        q = np.array([[int(v0), int(v1)]], dtype=np.int8)
        packed = orc.pack_int4(q)
        assert packed.shape == (1, 1) and packed[0, 0] == int(byte, 16)
        assert orc.dec_int4([packed[0, 0] & 0xF])[0] == int(v0)
        assert orc.dec_int4([packed[0, 0] >> 4])[0] == int(v1)


def test_f16_all_codes_match_numpy(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.lib().orc_dec_f16(int(b)) for b in bits])
    _same(got, ref)


def test_enc_f16_matches_numpy(orc):
    g = np.random.Generator(np.random.PCG64(5))
    vals = np.concatenate([
        g.standard_normal(4000) * 10.0 ** g.integers(-9, 6, 4000),
        np.ldexp(g.integers(0, 4096, 2000) + 0.5, -24 - 1),     # ties in the subnormal range
        np.ldexp(g.integers(1024, 2048, 2000) + 0.5, -10),      # ties in [1, 2)
        [65504.0, 65519.9, 65520.0, 65536.0, 1e6, 6e-8, 5.9604644775390625e-08, 2.98e-8, 0.0, -0.0],
    ])
    for v in vals:
        ref = int(np.array([v], dtype=np.float64).astype(np.float16).view(np.uint16)[0])
        assert orc.enc_f16(v) == ref, v
