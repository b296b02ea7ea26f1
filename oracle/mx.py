"""Decoding of the MX numbers the layer consumes (oracle side).

Test infrastructure: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use this package.

The pages name the formats (native MXFP4 weights: ktransformers issue
#2172, "Environment"; MXFP8 activations x MXFP4 weights: "Kimi-K3 SM120
FlashInfer MXFP4 MoE", goal section) but do not define them.  The
definitions written out here are those of the OCP Microscaling Formats
(MX) Specification v1.0 [external]:

* FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent field 0
  is subnormal (0 or 0.5); no Inf/NaN; max 6.0.
* FP8 E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field
  0 is subnormal (m/8 * 2**-6); S.1111.111 is NaN; no Inf; max 448.
* E8M0 scale: an unsigned biased exponent, value 2**(b-127); 0xFF is NaN.
* An MX block is 32 elements sharing one scale: value = scale * element.

Packed FP4 bytes hold element 2j in the low nibble and 2j+1 in the high
nibble (the pages only say the weights are handled as packed bytes).
Blocks run along the contiguous last axis, the reduction axis of the GEMM.

Everything is returned in float64.
"""
from __future__ import annotations

import numpy as np


def e2m1_value(code):
    """FP4 E2M1 code(s) 0..15 -> float64."""
    c = np.asarray(code, dtype=np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(s == 1, -mag, mag).astype(np.float64)


def e8m0_value(b):
    """E8M0 byte(s) -> float64 2**(b-127); 255 -> NaN."""
    b = np.asarray(b, dtype=np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)


def e4m3_value(code):
    """FP8 E4M3 byte(s) -> float64; S.1111.111 -> NaN."""
    c = np.asarray(code, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def bf16_value(bits):
    """bf16 bit patterns (uint16 / int16) -> float64 (the upper half of an fp32)."""
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# lookup tables built from the closed forms above
E2M1_TABLE = e2m1_value(np.arange(16))
E4M3_TABLE = e4m3_value(np.arange(256))
E8M0_TABLE = e8m0_value(np.arange(256))


def unpack_fp4(packed):
    """[..., K/2] uint8 -> [..., K] codes: element 2j = low nibble, 2j+1 = high nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def dequant_mxfp4(packed, scales):
    """MXFP4 matrix [N][K/2] + E8M0 [N][K/32] -> float64 [N][K].

    W[n][kk] = E2M1(code[n][kk]) * 2**(scale[n][kk // 32] - 127).
    """
    codes = unpack_fp4(packed)
    N, K = codes.shape[-2], codes.shape[-1]
    s = np.asarray(scales, dtype=np.uint8)
    if s.shape[-1] * 32 != K:
        raise ValueError("scale count does not match K/32")
    vals = E2M1_TABLE[codes].reshape(codes.shape[:-1] + (K // 32, 32))
    return (vals * E8M0_TABLE[s][..., None]).reshape(codes.shape)


def dequant_mxfp8(codes, scales):
    """MXFP8 E4M3 [T][K] + E8M0 [T][K/32] -> float64 [T][K]."""
    c = np.asarray(codes, dtype=np.uint8)
    s = np.asarray(scales, dtype=np.uint8)
    K = c.shape[-1]
    vals = E4M3_TABLE[c].reshape(c.shape[:-1] + (K // 32, 32))
    return (vals * E8M0_TABLE[s][..., None]).reshape(c.shape)


# --- MXFP8 encoding of the layer's intermediate ------------------------------
# The pages leave the precision of the SwiGLU output fed to FC2 open; the
# MXFP8 x MXFP4 product they describe ("Kimi-K3 SM120 FlashInfer MXFP4 MoE",
# goal section) is read as taking MXFP8 operands on both GEMMs.  The block
# scale is chosen so that no element saturates: the smallest exponent X with
# amax * 2**-X <= 448, the E4M3 maximum.  Elements round to the nearest E4M3
# value, ties to the even code (the OCP specification's default rounding).

_E4M3_POS = E4M3_TABLE[:127]   # codes 0x00..0x7E: the finite non-negative values, ascending


def mxfp8_block_exponent(amax):
    """Smallest integer X with amax * 2**-X <= 448, clamped to [-127, 127]; amax == 0 -> -127."""
    amax = float(amax)
    if not amax > 0.0:
        return -127
    x = int(np.ceil(np.log2(amax / 448.0)))
    # settle the floating-point guess against the exact power-of-two test
    while np.ldexp(amax, -x) > 448.0:
        x += 1
    while np.ldexp(amax, -(x - 1)) <= 448.0:
        x -= 1
    return max(-127, min(127, x))


def e4m3_nearest(v):
    """float64 value(s) with |v| <= 448 -> nearest E4M3 code, ties to the even code."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 126)   # first value >= a
    lo = np.clip(hi - 1, 0, 126)
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.int64)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def quantize_mxfp8(values):
    """[..., K] values (K % 32 == 0) -> (E4M3 codes [..., K], E8M0 bytes [..., K/32])."""
    v = np.asarray(values, dtype=np.float64)
    K = v.shape[-1]
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    blocks = v.reshape(-1, K // 32, 32)
    codes = np.empty(blocks.shape, dtype=np.uint8)
    scales = np.empty(blocks.shape[:2], dtype=np.uint8)
    for i in range(blocks.shape[0]):
        for b in range(blocks.shape[1]):
            x = mxfp8_block_exponent(np.max(np.abs(blocks[i, b])))
            scales[i, b] = x + 127
            codes[i, b] = e4m3_nearest(np.ldexp(blocks[i, b], -x))
    return codes.reshape(v.shape), scales.reshape(v.shape[:-1] + (K // 32,))
