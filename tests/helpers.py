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


def code_ulp_diff(a, b) -> np.ndarray:
    return np.abs(code_index(a) - code_index(b))


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
