"""Dequantization of the "FP8 with scale" KV cache row, written from its definition.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Row format (upstream FlashMLA README embedded in the DeepLink-org/
flashmla-optimization page, "FP8 KV Cache"): 656 bytes per token,

* bytes   0..511: 512 float8 e4m3 values, the quantized NoPE part;
* bytes 512..527: 4 float32 scales, scale g for values 128 g .. 128 g + 127;
* bytes 528..655: 64 bfloat16 values, the RoPE part, not quantized.

The kernel dequantizes the cache to bfloat16 and computes attention in
bfloat16 (same section).  The pages do not spell out the e4m3 encoding or the
rounding of the dequantized value; the readings taken here:

* e4m3 is the OCP 8-bit "E4M3" encoding as PyTorch's ``float8_e4m3fn``: 1 sign
  bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
  the subnormals m/8 * 2^-6; S.1111.111 is NaN; there are no infinities, so
  the largest finite magnitude is 1.75 * 2^8 = 448.
* A dequantized NoPE value is ``bf16(fp32(value * scale))``: the product is
  rounded to float32, then to bfloat16, both to nearest even (a float32
  multiply followed by a float32 -> bfloat16 conversion).
* Scales and RoPE values are little-endian.
"""
from __future__ import annotations

import numpy as np

ROW_BYTES = 656
NOPE = 512
ROPE = 64
GROUP = 128  # values per scale


def e4m3_value(code: int) -> float:
    """Value of one e4m3 byte, from the bit fields."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def round_to_f32(x: np.ndarray) -> np.ndarray:
    """Round float64 values to float32 (nearest even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even on the dropped 16 bits),
    returned as float64.  NaN stays NaN."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    out = r.view(np.float32).astype(np.float64)
    return np.where(np.isnan(f), np.nan, out)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def dequant_rows(raw) -> np.ndarray:
    """FP8-with-scale rows [..., 656] uint8 -> the 576 dequantized values as float64."""
    r = np.ascontiguousarray(np.asarray(raw, dtype=np.uint8))
    assert r.shape[-1] == ROW_BYTES
    lead = r.shape[:-1]
    r = r.reshape(-1, ROW_BYTES)
    vals = E4M3_TABLE[r[:, :NOPE]]                                     # [n, 512]
    scales = r[:, NOPE:NOPE + 16].copy().view("<f4").astype(np.float64)  # [n, 4]
    prod = vals * np.repeat(scales, GROUP, axis=1)                     # exact in float64
    nope = round_f32_to_bf16(round_to_f32(prod))
    rope = bf16_bits_to_f64(r[:, NOPE + 16:].copy().view("<u2"))       # [n, 64]
    return np.concatenate([nope, rope], axis=1).reshape(*lead, NOPE + ROPE)
