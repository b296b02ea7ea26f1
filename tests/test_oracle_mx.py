"""Pins of the oracle's MX decoders (oracle/mx.py) against things other than itself."""
import math
import os
import sys
import types

import numpy as np
import pytest
import torch

from oracle import mx
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_fp4_reference():
    """torch's own E2M1 unpacked->fp32 helper (torch.testing internals), if importable."""
    if "expecttest" not in sys.modules:
        stub = types.ModuleType("expecttest")
        stub.TestCase = type("TestCase", (), {})
        sys.modules["expecttest"] = stub
    try:
        from torch.testing._internal import common_quantized as cq
        return cq._floatx_unpacked_to_f32
    except Exception:
        return None


def test_e2m1_matches_ocp_table():
    rows = []
    with open(os.path.join(GOLDEN, "e2m1_ocp_v1.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, bits, val = line.split()
                s, e, m = bits.split(".")
                rows.append((int(s + e + m, 2), float(val)))
    assert len(rows) == 8
    for code, val in rows:
        got = mx.e2m1_value(code)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), (code, got, val)


def test_e2m1_matches_torch_reference_exhaustive():
    ref = _torch_fp4_reference()
    if ref is None:
        pytest.skip("torch's E2M1 reference helper is not importable")
    r = ref(torch.arange(16, dtype=torch.uint8), 2, 1).double().numpy()
    got = mx.e2m1_value(np.arange(16))
    np.testing.assert_array_equal(got, r)
    np.testing.assert_array_equal(np.signbit(got), np.signbit(r))


def test_e2m1_structure():
    v = mx.e2m1_value(np.arange(16))
    # sign symmetry, strictly increasing magnitudes over codes 0..7
    np.testing.assert_array_equal(v[8:], -v[:8])
    assert np.all(np.diff(v[:8]) > 0)


def test_e4m3_matches_torch_exhaustive():
    codes = torch.arange(256, dtype=torch.uint8)
    r = codes.view(torch.float8_e4m3fn).double().numpy()
    got = mx.e4m3_value(np.arange(256))
    nan = np.isnan(r)
    assert np.array_equal(nan, np.isnan(got))
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    np.testing.assert_array_equal(got[~nan], r[~nan])
    assert np.nanmax(got) == 448.0


def test_e8m0_matches_torch_exhaustive():
    codes = torch.arange(256, dtype=torch.uint8)
    r = codes.view(torch.float8_e8m0fnu).double().numpy()
    got = mx.e8m0_value(np.arange(256))
    assert np.isnan(got[255]) and np.isnan(r[255])
    np.testing.assert_array_equal(got[:255], r[:255])


def test_e8m0_is_the_fp32_exponent_field():
    # for b in 1..254 the fp32 with exponent field b and zero mantissa is 2**(b-127)
    b = np.arange(1, 255, dtype=np.uint32)
    f = (b << 23).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(mx.e8m0_value(b), f)


def test_bf16_value_matches_torch():
    g = np.random.default_rng(0)
    x = torch.from_numpy(g.standard_normal(1000).astype(np.float32)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy()
    np.testing.assert_array_equal(mx.bf16_value(bits), x.double().numpy())


def test_unpack_fp4_byte_roundtrip():
    b = np.arange(256, dtype=np.uint8)
    c = mx.unpack_fp4(b[None, :])[0]
    assert c.shape == (512,) and c.max() <= 15
    # element 2j is the low nibble, 2j+1 the high nibble; every byte recoverable
    np.testing.assert_array_equal(c[0::2] + 16 * c[1::2], b)


def _brute_dequant_mxfp4(packed, scales):
    N, K2 = packed.shape
    out = np.empty((N, 2 * K2))
    for n in range(N):
        for kk in range(2 * K2):
            byte = int(packed[n, kk // 2])
            code = (byte >> 4) if kk % 2 else (byte & 15)
            out[n, kk] = float(mx.e2m1_value(code)) * 2.0 ** (int(scales[n, kk // 32]) - 127)
    return out


def test_dequant_mxfp4_bruteforce():
    g = np.random.default_rng(1)
    p = g.integers(0, 256, (5, 48), dtype=np.uint8)       # K = 96 -> 3 blocks
    s = g.integers(100, 140, (5, 3), dtype=np.uint8)
    np.testing.assert_array_equal(mx.dequant_mxfp4(p, s), _brute_dequant_mxfp4(p, s))


def test_dequant_scale_is_a_power_of_two_per_block():
    g = np.random.default_rng(2)
    p = g.integers(0, 256, (4, 32), dtype=np.uint8)       # K = 64 -> 2 blocks
    s = g.integers(121, 128, (4, 2), dtype=np.uint8)
    base = mx.dequant_mxfp4(p, s)
    s2 = s.copy()
    s2[:, 1] += 1
    d = mx.dequant_mxfp4(p, s2)
    np.testing.assert_array_equal(d[:, :32], base[:, :32])
    np.testing.assert_array_equal(d[:, 32:], 2 * base[:, 32:])
    nan = s.copy()
    nan[0, 0] = 255
    dn = mx.dequant_mxfp4(p, nan)
    assert np.all(np.isnan(dn[0, :32])) and not np.any(np.isnan(dn[0, 32:]))


def test_dequant_mxfp8_bruteforce():
    g = np.random.default_rng(3)
    c = g.integers(0, 256, (3, 64), dtype=np.uint8)
    c[c == 0x7F] = 0
    c[c == 0xFF] = 0
    s = g.integers(110, 140, (3, 2), dtype=np.uint8)
    ref = torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    ref = ref * np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)
    np.testing.assert_array_equal(mx.dequant_mxfp8(c, s), ref)


# ---- the input generator's MXFP8 quantiser (input preparation) against the decoder

def test_quantize_mxfp8_is_nearest_even_on_the_grid():
    g = np.random.default_rng(4)
    x = torch.from_numpy(g.standard_normal((16, 128)).astype(np.float32)).to(torch.bfloat16).float()
    x[0, :32] = 0.0                                           # all-zero block
    x[1, 5] = 1e-30                                           # tiny value in an otherwise normal block
    codes, scales = gen.quantize_mxfp8(x)
    grid = mx.e4m3_value(np.arange(256))
    finite = ~np.isnan(grid)
    gv, gc = grid[finite], np.arange(256)[finite]
    xv = x.double().numpy()
    for r in range(16):
        for b in range(4):
            blk = xv[r, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            X = (math.floor(math.log2(amax)) - 8) if amax > 0 else -127
            assert int(scales[r, b]) == X + 127
            for i, v in enumerate(blk):
                q = v * 2.0 ** -X
                c = int(codes[r, 32 * b + i])
                got = grid[c]
                if abs(q) >= 448:
                    assert got == math.copysign(448.0, q)
                    continue
                dist = np.abs(gv - q)
                best = dist.min()
                cands = gc[dist == best]
                assert abs(got - q) == best, (r, b, i, q, got)
                if len(set(grid[cands])) > 1:                 # a tie: even mantissa wins
                    assert (c & 1) == 0
    deq = mx.dequant_mxfp8(codes.numpy(), scales.numpy())
    assert np.all(deq[0, :32] == 0)


# ---- the oracle's MXFP8 encoder of the intermediate (no-saturation block scale)

def test_intermediate_encoder_round_trips_every_code_at_every_scale():
    """Every finite E4M3 value times 2**X, placed in a block whose amax pins X,
    encodes back to its own code and to scale byte X + 127."""
    grid = mx.e4m3_value(np.arange(256))
    finite = np.flatnonzero(~np.isnan(grid) & (np.arange(256) != 0x80))
    for X in (-127, -20, -8, 0, 5, 100):
        for start in range(0, len(finite), 31):
            cs = finite[start:start + 31]
            blk = np.zeros(32)
            blk[:len(cs)] = np.ldexp(grid[cs], X)
            blk[31] = np.ldexp(448.0, X)                 # amax = 448 * 2**X exactly
            codes, scales = mx.quantize_mxfp8(blk[None, :])
            assert int(scales[0, 0]) == X + 127
            assert np.array_equal(codes[0, :len(cs)], cs.astype(np.uint8)), X
            assert codes[0, 31] == 0x7E


def test_intermediate_encoder_scale_rule_and_ties():
    # amax just above 448 * 2**X needs the next exponent; just at it does not
    for X in (-10, 0, 7):
        at = np.full((1, 32), np.ldexp(448.0, X))
        above = at.copy()
        above[0, 3] = np.nextafter(np.ldexp(448.0, X), np.inf)
        assert mx.quantize_mxfp8(at)[1][0, 0] == X + 127
        assert mx.quantize_mxfp8(above)[1][0, 0] == X + 128
    # an all-zero block: smallest scale, zero codes; a negative zero keeps its sign
    z = np.zeros((1, 32))
    z[0, 5] = -0.0
    codes, scales = mx.quantize_mxfp8(z)
    assert scales[0, 0] == 0 and codes[0, 0] == 0 and codes[0, 5] == 0x80
    # midpoints between neighbouring codes go to the even code (amax 448 pins X = 0)
    grid = mx.e4m3_value(np.arange(0x7F))
    for c in range(0, 0x7E):
        mid = (grid[c] + grid[c + 1]) / 2
        blk = np.array([[mid, -mid] + [0.0] * 29 + [448.0]])
        codes, _ = mx.quantize_mxfp8(blk)
        even = c if c % 2 == 0 else c + 1
        assert codes[0, 0] == even and codes[0, 1] == (even | 0x80), c


def test_intermediate_encoder_is_within_half_an_ulp():
    g = np.random.default_rng(11)
    v = g.standard_normal((8, 96)) * np.exp(g.uniform(-6, 6, (8, 1)))
    codes, scales = mx.quantize_mxfp8(v)
    back = mx.dequant_mxfp8(codes, scales)
    # E4M3 has 3 mantissa bits: relative error <= 2**-4 for normals; subnormals
    # are absolute multiples of 2**-9 of the block scale
    sc = np.repeat(mx.e8m0_value(scales), 32, axis=1)
    err = np.abs(back - v)
    assert np.all(err <= np.maximum(np.abs(v) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 1e-12))
