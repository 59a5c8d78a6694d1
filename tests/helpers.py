"""Small test-side helpers: code distances, bf16 decoding, golden-file parsing."""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def code_index(c) -> np.ndarray:
    """Signed position of an e4m3fn code on the value line (+0 and -0 both 0).

    Finite codes 0x00..0x7E increase in magnitude with the code, so two codes
    are one ULP apart exactly when their indices differ by one."""
    c = np.asarray(c, dtype=np.uint8).astype(np.int16)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


# Distance given to a position where exactly one side is a NaN code: no
# finite number of ULPs, so it fails every bar.
NAN_MISMATCH = 1 << 10


def is_nan_code(c) -> np.ndarray:
    """e4m3fn NaN codes (0x7F and 0xFF; the format has no infinities)."""
    return (np.asarray(c, dtype=np.uint8) & 0x7F) == 0x7F


def code_ulp_diff(a, b) -> np.ndarray:
    """Distance in ULPs between e4m3fn codes, position by position.

    Two NaN codes are equal (whatever their sign bits); a NaN against any
    finite code counts as NAN_MISMATCH, so a NaN where the other side has
    +-448 is never taken for the neighbouring code.  Finite codes are compared
    by their positions on the value line (+0 and -0 both 0)."""
    na, nb = is_nan_code(a), is_nan_code(b)
    d = np.abs(code_index(a) - code_index(b))
    d = np.where(na & nb, 0, d)
    return np.where(na ^ nb, NAN_MISMATCH, d)


def bf16_to_f64(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_torch(a) -> np.ndarray:
    """float64 -> float32 -> bf16 via torch (a library rounding, for pins)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return t.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def torch_e4m3fn(a) -> np.ndarray:
    """Values with |a| <= 448 -> e4m3fn codes via torch's conversion.

    torch converts float64 through float32, so the result is a single rounding
    only for float32-representable inputs or inputs far from an e4m3 midpoint."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def read_kv(name: str) -> dict:
    """Parse a golden file of 'key value...' lines (# starts a comment)."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


def read_rows(name: str) -> list:
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


# Exact ties through the whole op.  A row whose only nonzero is z0, with
# eps = 1 - z0^2 / H, has mean(z^2) + eps = 1 and so rho = 1 exactly; with
# weight w0 its output is y0 = z0 * w0 exactly, and the static scale s is
# chosen so that y0 / s is exactly the midpoint m between two adjacent e4m3fn
# values.  The code must then be the one with the even mantissa (round to
# nearest, ties to even, of the exact quotient).  For every s below the double
# reciprocal of s is inexact enough that y0 * (1/s) misses m (the last column
# says to which side), so a quotient taken by a reciprocal fails this pin.
# Columns: s, m, z0, w0, eps, the expected code, side of y0 * (1/s).
TIE_CASES = [
    (1.095703125, 0.0009765625, 0.0029296875, 0.365234375, 0.999998927116394, 0, "down"),
    (1.171875, 0.0068359375, 0.0029296875, 2.734375, 0.999998927116394, 4, "up"),
    (1.736328125, 0.0185546875, 0.1240234375, 0.259765625, 0.9980772733688354, 10, "up"),
    (1.416015625, 0.048828125, 0.1220703125, 0.56640625, 0.998137354850769, 20, "down"),
    (1.921875, 0.265625, 0.0166015625, 30.75, 0.9999655485153198, 40, "up"),
    (1.416015625, 1.5625, 0.1220703125, 18.125, 0.998137354850769, 60, "down"),
    (1.921875, 8.5, 0.0166015625, 984.0, 0.9999655485153198, 80, "up"),
    (1.416015625, 50.0, 0.1220703125, 580.0, 0.998137354850769, 100, "down"),
    (1.421875, 184.0, 0.0126953125, 20608.0, 0.9999798536300659, 116, "up"),
]


def e4m3_value(code: int) -> float:
    """Value of a non-negative e4m3fn code from the format definition."""
    e, m = code >> 3, code & 7
    return m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
