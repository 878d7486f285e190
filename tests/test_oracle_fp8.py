"""Pins of the FP8-with-scale dequantization in the oracle (``oracle.fp8``).

The row format is the upstream FlashMLA README's "FP8 KV Cache" section: 512
e4m3 values, 4 fp32 scales (one per 128 values), 64 bf16 RoPE values.

* e4m3 decoding: every one of the 256 codes against PyTorch's float8_e4m3fn
  conversion (a library routine), and the format's landmark values.
* bf16 rounding: against PyTorch's float32 -> bfloat16 conversion, including
  exact ties (both directions), NaN, infinities and overflow.
* Row layout: a row assembled byte by byte; scale g must scale exactly values
  128 g .. 128 g + 127, and the RoPE part must come through unchanged.
* Power-of-two scales: the dequantized value is the exact product (closed form:
  no rounding happens), for every code.
* A decode over an FP8 cache equals the decode over the bf16 cache holding the
  dequantized rows, dense and sparse (the dequantization is the only
  difference between the two formats).
"""
import struct

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8


def test_e4m3_table_matches_library_for_every_code():
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = fp8.E4M3_TABLE
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    assert np.array_equal(ours[~np.isnan(ours)], lib[~np.isnan(lib)])


def test_e4m3_landmarks():
    t = fp8.E4M3_TABLE
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and np.signbit(t[0x80])
    assert t[0x01] == 2.0 ** -9            # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert t[0x08] == 2.0 ** -6            # smallest normal
    assert t[0x38] == 1.0 and t[0xB8] == -1.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0  # largest finite
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isnan(t).sum() == 2 and not np.isinf(t).any()


def test_bf16_rounding_matches_library():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000),
        # exact ties: the low 16 bits are 0x8000, kept bit even and odd
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([np.inf, -np.inf, 3.4e38, -3.4e38, 1e-40, -1e-45, 0.0, -0.0], dtype=np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    ours = fp8.round_f32_to_bf16(x)
    assert np.array_equal(ours, ref)
    assert np.isnan(fp8.round_f32_to_bf16(np.array([np.nan], np.float32)))[0]


def _row(codes, scales, rope_bits):
    return np.frombuffer(bytes(codes) + struct.pack("<4f", *scales)
                         + struct.pack("<64H", *rope_bits), dtype=np.uint8)


def test_row_layout_scale_groups_and_rope_passthrough():
    codes = [0x38] * 512  # all 1.0
    scales = [2.0, 0.5, -3.0, 0.125]
    rope_bits = [0x3F80 + i for i in range(64)]  # 1.0, then the next bf16 values up
    row = _row(codes, scales, rope_bits)
    assert row.size == fp8.ROW_BYTES
    d = fp8.dequant_rows(row[None])[0]
    assert d.shape == (576,)
    for g in range(4):
        assert np.all(d[128 * g:128 * (g + 1)] == scales[g])
    want_rope = np.array([struct.unpack("<f", struct.pack("<I", b << 16))[0] for b in rope_bits])
    assert np.array_equal(d[512:], want_rope)


def test_power_of_two_scales_are_exact_for_every_code():
    for k in (-12, -3, 0, 5):
        codes = list(range(256)) * 2
        row = _row(codes, [2.0 ** k] * 4, [0] * 64)
        d = fp8.dequant_rows(row[None])[0][:512]
        want = np.tile(fp8.E4M3_TABLE, 2) * 2.0 ** k
        fin = ~np.isnan(want)
        assert np.array_equal(d[fin], want[fin]) and np.all(np.isnan(d[~fin]))


def test_general_scale_rounds_once_to_f32_then_to_bf16():
    # 1.125 * 0.3f: exact product, its float32 rounding, then bfloat16
    s = np.float32(0.3)
    row = _row([0x39] + [0] * 511, [float(s), 1.0, 1.0, 1.0], [0] * 64)
    got = fp8.dequant_rows(row[None])[0][0]
    prod32 = np.float32(np.float32(1.125) * s)
    want = torch.tensor(float(prod32), dtype=torch.float32).to(torch.bfloat16).item()
    assert got == want


def _fp8_cache(rng, n_rows):
    """Random well-formed FP8 rows (no NaN codes) and their dequantized values."""
    codes = rng.integers(0, 256, size=(n_rows, 512)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E
    scales = (rng.lognormal(-5, 1, size=(n_rows, 4))).astype(np.float32)
    rope = torch.from_numpy(rng.standard_normal((n_rows, 64)).astype(np.float32)).to(torch.bfloat16)
    raw = np.concatenate([codes, scales.view(np.uint8).reshape(n_rows, 16),
                          rope.view(torch.int16).numpy().view(np.uint8).reshape(n_rows, 128)], axis=1)
    return raw, fp8.dequant_rows(raw)


def test_decode_over_fp8_cache_equals_decode_over_dequantized_cache():
    rng = np.random.default_rng(11)
    B, s_q, h_q, pool = 3, 2, 8, 6
    raw, deq = _fp8_cache(rng, pool * 64)
    kv8 = torch.from_numpy(raw.reshape(pool, 64, 1, 656))
    kv64 = torch.from_numpy(deq.reshape(pool, 64, 1, 576))
    q = torch.from_numpy(rng.standard_normal((B, s_q, h_q, 576)))
    bt = torch.tensor([[0, 3], [5, 1], [2, 4]], dtype=torch.int32)
    sl = torch.tensor([100, 64, 7], dtype=torch.int32)
    o8, l8 = oracle.ref_decode_paged(q, kv8, bt, sl, 512, True, 576 ** -0.5)
    o, l = oracle.ref_decode_paged(q, kv64, bt, sl, 512, True, 576 ** -0.5)
    assert np.array_equal(o8, o) and np.array_equal(l8, l)
    idx = torch.from_numpy(rng.integers(-5, pool * 64, size=(B, s_q, 40)).astype(np.int32))
    o8, l8 = oracle.ref_decode_sparse(q, kv8, idx, 512, 0.05)
    o, l = oracle.ref_decode_sparse(q, kv64, idx, 512, 0.05)
    assert np.array_equal(o8, o) and np.array_equal(l8, l)
