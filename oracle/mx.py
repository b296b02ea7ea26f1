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
