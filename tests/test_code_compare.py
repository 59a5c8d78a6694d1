"""The code-comparison rule that the GPU parity tests and smoke() use, on the
CPU: adjacent finite codes are one ULP apart, +0 and -0 are equal, two NaN
codes are equal, and a NaN code against any finite code (448 included, the
code next to NaN in bit order) fails outright."""
import os
import sys

import numpy as np

from gpu_util import CODE_MISMATCH_BUDGET
from helpers import NAN_MISMATCH, code_ulp_diff

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_finite_codes_by_value_line():
    a = np.array([0x00, 0x80, 0x7E, 0x7D, 0x01, 0x81, 0x38], np.uint8)
    b = np.array([0x80, 0x00, 0x7D, 0x7E, 0x81, 0x01, 0x39], np.uint8)
    assert code_ulp_diff(a, b).tolist() == [0, 0, 1, 1, 2, 2, 1]


def test_nan_codes():
    a = np.array([0x7F, 0xFF, 0x7F, 0x7E, 0xFF, 0xFE], np.uint8)
    b = np.array([0xFF, 0x7F, 0x7E, 0x7F, 0xFE, 0xFF], np.uint8)
    d = code_ulp_diff(a, b)
    assert d.tolist() == [0, 0, NAN_MISMATCH, NAN_MISMATCH, NAN_MISMATCH, NAN_MISMATCH]
    assert NAN_MISMATCH > 1


def test_smoke_check_rejects_one_sided_nan():
    import __graft_entry__ as g

    ref = np.full(100000, 0x7E, np.uint8)
    gpu = ref.copy()
    assert g._codes_ok(gpu, ref)
    gpu[3] = 0x7D  # one ULP, within the 1e-4 budget
    assert g._codes_ok(gpu, ref)
    gpu[5] = 0x7F  # NaN where the oracle has 448
    assert not g._codes_ok(gpu, ref)
    both = ref.copy()
    both[7] = 0xFF
    ref2 = ref.copy()
    ref2[7] = 0x7F  # NaN on both sides (sign bits differ)
    assert g._codes_ok(both, ref2)
    many = ref.copy()
    many[: int(CODE_MISMATCH_BUDGET * many.size) + 2] = 0x7D
    assert not g._codes_ok(many, ref)
