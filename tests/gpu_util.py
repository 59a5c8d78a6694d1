"""Helpers for the GPU parity tests: host <-> device transfer of bit patterns
and the acceptance bars.

Bars: FP8 codes may differ from the oracle by at most one code (adjacent
values) on at most 1e-4 of all codes; bf16 outputs and fp32 scales within
rtol 1e-2 (bf16 outputs also atol 1e-5, for values that cancel to near zero);
fp16 outputs within one fp16 unit of the oracle (plus 2^-20 absolute);
integer and index work (which slots are written, bit copies) bit-exact."""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import pytest

from helpers import bf16_to_f64, code_ulp_diff

CODE_MISMATCH_BUDGET = 1e-4
RTOL = 1e-2
ATOL_BF16 = 1e-5


def torch_mod():
    import torch

    return torch


def require_gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(msg: str) -> None:
    """Name the case on stdout before it touches the GPU."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f16(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.float16).cuda()


def dev_elem(a: np.ndarray, dtype: str):
    """uint16 bit patterns -> a device tensor of element type dtype ("bf16"/"f16")."""
    return dev_f16(a) if dtype == "f16" else dev_bf16(a)


def dev(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bf16(t) -> np.ndarray:
    """16-bit device tensor (bf16 or fp16) -> its uint16 bit patterns."""
    torch = torch_mod()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t) -> np.ndarray:
    torch = torch_mod()
    return t.contiguous().view(torch.uint8).cpu().numpy()


def host_f32(t) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def assert_codes(gpu: np.ndarray, ref: np.ndarray, what: str, exact: bool = False) -> dict:
    """FP8 codes against the oracle's.  exact: every code must be the oracle's
    (the norm kernels round each code as the exact quotient would).
    Otherwise (SiLU, whose activation is formed in fp32) codes may differ by
    one code on at most CODE_MISMATCH_BUDGET of them; a case of fewer codes
    than 1 / CODE_MISMATCH_BUDGET may have one, the least whole count that
    fraction can mean at that size."""
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    d = code_ulp_diff(gpu, ref)
    n = d.size
    bad = int(np.count_nonzero(d))
    stats = dict(what=what, codes=n, mismatches=bad, max_ulp=int(d.max()) if n else 0)
    print(stats, flush=True)
    _record("codes", stats)
    if exact:
        assert bad == 0, stats
    assert stats["max_ulp"] <= 1, stats
    assert bad <= max(1.0, CODE_MISMATCH_BUDGET * n), stats
    return stats


def assert_scales(gpu: np.ndarray, ref: np.ndarray, what: str) -> None:
    assert gpu.shape == ref.shape
    ok = np.isclose(gpu.astype(np.float64), ref.astype(np.float64), rtol=RTOL, atol=0)
    assert ok.all(), (what, np.argwhere(~ok)[:5])
    exact = np.mean(gpu.view(np.uint32) == ref.view(np.uint32)) if gpu.size else 1.0
    stats = dict(what=what, scales=gpu.size, bit_exact_fraction=float(exact))
    print(stats, flush=True)
    _record("scales", stats)


def assert_bf16(gpu: np.ndarray, ref: np.ndarray, what: str) -> None:
    assert gpu.shape == ref.shape
    g, r = bf16_to_f64(gpu), bf16_to_f64(ref)
    ok = np.isclose(g, r, rtol=RTOL, atol=ATOL_BF16)
    assert ok.all(), (what, np.argwhere(~ok)[:5], g[~ok][:5], r[~ok][:5])
    exact = float(np.mean(gpu == ref)) if gpu.size else 1.0
    stats = dict(what=what, values=gpu.size, bit_exact_fraction=exact)
    print(stats, flush=True)
    _record("bf16", stats)


# fp16 results: the kernels compute in fp32 and round once, the oracle in
# double; the two may straddle a rounding point (one fp16 unit apart) and, where
# a rotation cancels, differ by fp32 rounding of the products (absolute 2^-20
# covers |inputs| up to 16).
ATOL_F16 = 2.0 ** -20


def _f16_ulp(r: np.ndarray) -> np.ndarray:
    e = np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -14)))
    return np.exp2(e - 10)


def assert_f16(gpu: np.ndarray, ref: np.ndarray, what: str) -> None:
    assert gpu.shape == ref.shape
    g = gpu.view(np.float16).astype(np.float64)
    r = ref.view(np.float16).astype(np.float64)
    ok = np.abs(g - r) <= _f16_ulp(r) + ATOL_F16
    assert ok.all(), (what, np.argwhere(~ok)[:5], g[~ok][:5], r[~ok][:5])
    exact = float(np.mean(gpu == ref)) if gpu.size else 1.0
    stats = dict(what=what, values=gpu.size, bit_exact_fraction=exact)
    print(stats, flush=True)
    _record("f16", stats)


def assert_elem(gpu: np.ndarray, ref: np.ndarray, what: str, dtype: str) -> None:
    (assert_f16 if dtype == "f16" else assert_bf16)(gpu, ref, what)


def compare_rows(T: int) -> np.ndarray:
    """Row (token) indices compared element by element with the oracle: every
    row, at every size the tests run (the oracle computes T = 16384 rows of any
    kernel in a few seconds)."""
    return np.arange(T)


def _record(kind: str, stats: dict) -> None:
    """Append one comparison's measured figures to the JSON-lines file named by
    RRA_PARITY_LOG (when set), tagged with the running test, for the committed
    parity summary (tests/parity_summary.py)."""
    path = os.environ.get("RRA_PARITY_LOG")
    if not path:
        return
    rec = dict(stats, kind=kind, test=os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0])
    with open(path, "a", encoding="utf-8") as f:
        f.write(json.dumps(rec) + "\n")
