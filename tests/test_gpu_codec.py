"""GPU pack (quantise) and unpack (dequantise) against the oracle: bit-exact on every output."""
import numpy as np
import pytest
import torch

from block_scaled_quantized_amd import synth
from gpu_common import bitequal_f32, dev, empty, sentinel_f32, gpu_int_pack, gpu_mx_pack, host, require_gpu, say

pytestmark = pytest.mark.gpu


def edge_rows(cols, seed):
    x = synth.normal((24, cols), 1.0, seed)
    x[0] = 0.0
    x[1, :32] = -0.0
    x[2] *= np.float32(1e-40)                      # subnormal fp32 sources
    x[3] *= np.float32(3e37)                       # blocks near the fp32 top
    x[4, 5] = np.inf
    x[5, 40] = np.nan
    x[6, :32] = np.float32(2.0) ** np.arange(-16, 16, dtype=np.float32)
    x[7] = np.float32(1344.0) * np.sign(x[7])      # saturating elements
    x[8, :32] = np.float32(2.0) ** np.float32(-130)  # amax below 2^-127: scale clamps to 0
    x[9, 32:64] = -np.inf
    # exact ties of the element grids after scaling (block amax 448 -> scale 2^0 for E4M3)
    grid = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    mids = (grid[:-1] + grid[1:]) / 2
    x[10, :32] = np.float32(448.0)
    x[10, 1:32] = mids[np.linspace(0, len(mids) - 1, 31).astype(int)]
    x[12, :32] = -x[10, :32]
    x[13, :32] = np.float32(57344.0)               # E5M2 block amax 57344 -> scale 2^0: its ties
    e5 = torch.arange(0x7C, dtype=torch.uint8).view(torch.float8_e5m2).float().numpy()
    x[13, 1:32] = ((e5[:-1] + e5[1:]) / 2)[np.linspace(0, len(e5) - 2, 31).astype(int)]
    x[14, :32] = np.float32(60000.0) * np.sign(x[14, :32])   # E5M2 saturation
    x[11, :32] = np.float32(4.0)                   # E2M1 block amax 4 -> scale 2^0
    x[11, 1:16] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5,
                            -3.5, -5.0, 0.1], np.float32)
    return x.astype(np.float32)



def every_scale_blocks(fmt, nblocks, seed):
    """Blocks of 32 fp32 values: block b's first element sets the block's scale code to b % 255, or
    to the largest code a finite fp32 amax reaches (127 - emax + 127: 246 for E4M3, emax 8; 252
    for E2M1, emax 2). The other 31 are random bit patterns (sign, 23-bit mantissa) with
    exponents from the amax's down 50 binades (fp32 subnormals where that reaches below 2^-126),
    so their scaled values sweep every element grid point and the round-off between them."""
    emax = 8 if fmt == 0 else 2
    g = synth.rng(seed)
    E = np.arange(nblocks) % 255
    ex_amax = np.clip(E + emax, 0, 254)                          # biased fp32 exponent of the amax
    ex = ex_amax[:, None] - g.integers(0, 51, size=(nblocks, 32))
    ex[:, 0] = ex_amax
    ex = np.clip(ex, 0, 254).astype(np.uint32)
    man = g.integers(0, 1 << 23, size=(nblocks, 32), dtype=np.uint32)
    man[:, 0] |= np.uint32(1 << 22) * (g.integers(0, 2, size=nblocks, dtype=np.uint32))
    sign = g.integers(0, 2, size=(nblocks, 32), dtype=np.uint32) << np.uint32(31)
    bits = sign | (ex << np.uint32(23)) | man
    return bits.view(np.float32).reshape(nblocks // 64, 64 * 32)


@pytest.mark.parametrize("fmt", [0, 4])
def test_mx_pack_every_scale_code(orc, fmt):
    """The E4M3 and E2M1 packs (gfx950's scaled conversions) against the oracle's quantiser on
    blocks that set every scale code a finite fp32 block can have, bit for bit."""
    api = require_gpu()
    x = every_scale_blocks(fmt, 1 << 16, 3300 + fmt)
    rows, cols = x.shape
    say(f"mx pack every scale code fmt={fmt} {rows}x{cols}")
    codes, scales = gpu_mx_pack(api, fmt, x)
    oc, os_ = orc.mx_quantize(fmt, x)
    top = 127 - (8 if fmt == 0 else 2) + 127
    assert np.array_equal(np.unique(os_), np.arange(top + 1, dtype=np.uint8))
    assert np.array_equal(host(scales), os_)
    assert np.array_equal(host(codes), oc)

@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("case", ["normal1", "normal002", "edges", "prefill_rows"])
def test_mx_pack_unpack_bitexact(orc, fmt, case):
    api = require_gpu()
    say(f"mx pack fmt={fmt} case={case}")
    if case == "normal1":
        x = synth.normal((384, 512), 1.0, 1000)
    elif case == "normal002":
        x = synth.normal((256, 1024), 0.02, 1021)
    elif case == "edges":
        x = edge_rows(256, 7)
    else:
        x = synth.normal((64, 4096), 1.0, 1020)
    rows, cols = x.shape
    codes, scales = gpu_mx_pack(api, fmt, x)
    oc, os_ = orc.mx_quantize(fmt, x)
    assert np.array_equal(host(scales), os_)
    assert np.array_equal(host(codes), oc)
    out = sentinel_f32((rows, cols))
    api.mx_unpack_run(fmt, codes, scales, rows, cols, out)
    assert bitequal_f32(host(out), orc.dequant(fmt, oc, os_, rows, cols))


@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
def test_mx_unpack_every_code_and_scale(orc, fmt):
    api = require_gpu()
    say(f"mx unpack exhaustive fmt={fmt}")
    # every code byte against every scale byte: 256 rows (one per scale) x 256 or 512 columns
    byte = fmt in (0, 1)
    cols = 256 if byte else 512
    per_row = np.arange(256, dtype=np.uint8)
    codes = np.tile(per_row, (256, 1))
    if fmt in (2, 3):   # every 6-bit code, 8 times per row, packed as the little-endian bit stream
        fields = np.tile(np.arange(64, dtype=np.uint8), cols // 64)
        bits = ((fields[:, None] >> np.arange(6)) & 1).astype(np.uint8).reshape(-1)
        codes = np.tile(np.packbits(bits, bitorder="little"), (256, 1))
    codes = np.ascontiguousarray(codes[:, : (cols if byte else (cols // 4 * 3 if fmt in (2, 3) else cols // 2))])
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], cols // 32, axis=1)
    out = sentinel_f32((256, cols))
    api.mx_unpack_run(fmt, dev(codes), dev(scales), 256, cols, out)
    assert bitequal_f32(host(out), orc.dequant(fmt, codes, scales, 256, cols))


@pytest.mark.parametrize("fw", [32, 33])
@pytest.mark.parametrize("shape", [(4096, 14336), (96, 48), (64, 34)])
def test_int_pack_unpack_bitexact(orc, fw, shape):
    api = require_gpu()
    K, N = shape
    if fw == 33 and N % 2:
        pytest.skip("int4 needs an even column count")
    say(f"int pack fw={fw} K={K} N={N}")
    w = synth.normal((K, N), 0.02, 1031)
    if K <= 96:
        w[32:64, 3] = 0.0
        w[0:32, 5] *= np.float32(1e-30)
        w[40, 6] = np.inf                    # non-finite blocks: NaN scale, zero codes
        w[45, 7] = np.nan
        w[2, 8] = -np.inf
    codes, scales = gpu_int_pack(api, fw, w)
    q, s = orc.int_quantize(fw, w)
    ref_codes = q.view(np.uint8) if fw == 32 else orc.pack_int4(q)
    assert np.array_equal(host(scales).view(np.uint16), s.view(np.uint16))
    assert np.array_equal(host(codes), ref_codes)
    out = sentinel_f32((K, N))
    api.mx_unpack_run(fw, codes, scales, K, N, out)
    assert bitequal_f32(host(out), orc.dequant(fw, ref_codes, s, K, N))
