"""Pins for the oracle's bf16 and e4m3fn codecs.

The oracle's encoders are checked against the OCP E4M3 definition (golden
table), against torch's independent float8/bfloat16 conversions, against each
other exhaustively over all 2^32 float32 bit patterns, and on hand-derived
rounding cases (ties to even, saturation, signed zero)."""
import math

import numpy as np
import pytest
import torch

from helpers import read_rows, torch_e4m3fn


def _structured_f32() -> np.ndarray:
    """Every sign/exponent/top-7-mantissa combination, each with low 16 bits
    chosen to sit on, just below and just above the rounding points of both
    bf16 (bit 15) and e4m3fn (bits 19 and below)."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x3FFF, 0xC000],
                    dtype=np.uint32)
    return (hi[:, None] | lows[None, :]).ravel().view(np.float32)


def test_e4m3fn_ocp_table(oracle):
    for code_s, val_s in read_rows("e4m3fn_ocp.txt"):
        code, val = int(code_s, 16), float(val_s)
        d = oracle.e4m3fn_decode(code)
        if math.isnan(val):
            assert math.isnan(d)
            continue
        assert d == val and math.copysign(1, d) == math.copysign(1, val), hex(code)
        assert oracle.e4m3fn_encode(val) == code, hex(code)
        assert oracle.e4m3fn_encode_arith(val) == code, hex(code)


def test_e4m3fn_value_line(oracle):
    vals = [oracle.e4m3fn_decode(c) for c in range(0x7F)]
    assert vals[0] == 0.0 and vals[-1] == 448.0
    assert all(b > a for a, b in zip(vals, vals[1:]))
    assert math.isnan(oracle.e4m3fn_decode(0x7F)) and math.isnan(oracle.e4m3fn_decode(0xFF))
    for c in range(0x7F):
        assert oracle.e4m3fn_decode(c | 0x80) == -vals[c]
        assert oracle.e4m3fn_encode(vals[c]) == c  # round trip


def test_e4m3fn_rounding_cases(oracle):
    enc = oracle.e4m3fn_encode
    # ties go to the even code
    assert enc(5.25) == 0x4A  # between 5.0 (0x4a) and 5.5 (0x4b)
    assert enc(5.75) == 0x4C  # between 5.5 (0x4b) and 6.0 (0x4c)
    assert enc(432.0) == 0x7E  # between 416 (0x7d) and 448 (0x7e)
    assert enc(7.5 * 2 ** -9) == 0x08  # largest subnormal | smallest normal
    assert enc(2 ** -10) == 0x00 and enc(1.5 * 2 ** -10) == 0x01
    # off-tie values go to the nearer neighbour
    assert enc(5.25 + 2 ** -40) == 0x4B and enc(5.25 - 2 ** -40) == 0x4A
    # saturation, signs, zeros
    for v in (448.0, 448.0 * (1 + 2 ** -24), 464.0, 480.0, 1e30, math.inf):
        assert enc(v) == 0x7E and enc(-v) == 0xFE
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80
    assert enc(math.nan) & 0x7F == 0x7F


def test_e4m3fn_encoders_agree_on_all_f32(oracle):
    assert oracle.e4m3fn_cross_check(0, 1 << 32) == 0


def test_e4m3fn_matches_torch(oracle):
    f = _structured_f32()
    f = f[np.isfinite(f) & (np.abs(f) <= 448.0)]
    ours = oracle.e4m3fn_encode_f32(f)
    ref = torch_e4m3fn(f.astype(np.float64))
    bad = np.flatnonzero(ours != ref)
    assert bad.size == 0, [(float(f[i]), hex(ours[i]), hex(ref[i])) for i in bad[:8]]


def test_bf16_matches_torch(oracle):
    f = _structured_f32()
    ours = oracle.bf16_encode_f32(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all(ours[nan] & 0x7F)


def test_bf16_double_rounding_cases(oracle):
    enc = oracle.bf16_encode
    assert enc(1.0 + 2 ** -8) == 0x3F80  # tie -> even (1.0)
    assert enc(1.0 + 2 ** -8 + 2 ** -40) == 0x3F81
    assert enc(1.0 + 3 * 2 ** -8) == 0x3F82  # tie -> even (1 + 2^-6)
    assert enc(-0.0) == 0x8000 and enc(0.0) == 0x0000
    assert enc(3.4e38) == 0x7F80 and enc(-1e300) == 0xFF80  # overflow
    assert enc(2 ** -133) == 0x0001  # smallest subnormal
    assert enc(2 ** -134) == 0x0000  # tie -> even (zero)
    for h in (0x0001, 0x3F80, 0x7F7F, 0xC2F7, 0x8001):
        assert enc(oracle.bf16_decode(h)) == h


def test_fp32_round(oracle):
    for v in (1 / 3, 1 / 448, 2.0 ** -140, 123456.789):
        assert oracle.fp32_round(v) == float(np.float32(v))


# ---- IEEE binary16 (fp16) -----------------------------------------------------

def _all_f16_values() -> np.ndarray:
    return np.arange(1 << 16, dtype=np.uint16).view(np.float16).astype(np.float64)


def test_f16_decode_matches_numpy_on_every_code(oracle):
    ref = _all_f16_values()
    ours = np.array([oracle.f16_decode(c) for c in range(1 << 16)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))  # -0.0


def test_f16_encode_matches_numpy_at_rounding_points(oracle):
    """Every finite positive fp16 value, the exact midpoint to its upper
    neighbour (a tie) and doubles a hair on either side of that midpoint, in
    both signs; numpy converts float64 -> float16 directly, with one rounding."""
    vals = _all_f16_values()[:0x7C00]  # +0 .. 65504
    mids = (vals[:-1] + vals[1:]) / 2
    top = np.array([65504.0 + 8, 65504.0 + 16, 65504.0 + 16 - 2 ** -30, 1e6])
    x = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf), top])
    x = np.concatenate([x, -x])
    ours = np.array([oracle.f16_encode(v) for v in x], np.uint16)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    bad = np.flatnonzero(ours != ref)
    assert bad.size == 0, [(float(x[i]), hex(ours[i]), hex(ref[i])) for i in bad[:8]]


def test_f16_rounding_cases(oracle):
    enc = oracle.f16_encode
    assert enc(1.0) == 0x3C00 and enc(-2.0) == 0xC000
    assert enc(1.0 + 2 ** -11) == 0x3C00  # tie -> even (1.0)
    assert enc(1.0 + 3 * 2 ** -11) == 0x3C02  # tie -> even (1 + 2^-9)
    assert enc(1.0 + 2 ** -11 + 2 ** -40) == 0x3C01
    assert enc(65504.0) == 0x7BFF  # largest finite
    assert enc(65519.99) == 0x7BFF and enc(65520.0) == 0x7C00  # tie at the top -> inf
    assert enc(-1e300) == 0xFC00 and enc(math.inf) == 0x7C00
    assert enc(2 ** -24) == 0x0001 and enc(2 ** -25) == 0x0000  # tie -> even (zero)
    assert enc(3 * 2 ** -25) == 0x0002  # tie between 1 and 2 units -> 2
    assert enc(2 ** -14 - 2 ** -25) == 0x0400  # largest subnormal rounds up to the smallest normal
    assert enc(-0.0) == 0x8000 and enc(0.0) == 0x0000
    assert (enc(math.nan) & 0x7C00) == 0x7C00 and (enc(math.nan) & 0x3FF)
    for h in (0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0xC2F7, 0x8001):
        assert enc(oracle.f16_decode(h)) == h
