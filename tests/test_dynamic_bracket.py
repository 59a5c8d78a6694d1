"""The bracket that the norm kernels use for codes with a dynamic scale.

With s = fp32(m * rho / 448) for a slice of amax m * rho (m = max |t|), the
exact quotient is q = t * rho / s = 448 t / (m (1 + e)), e the fp32 rounding of
s, so the kernels bracket every q of a slice with f_dn = fp32(f (1 - 2^-20))
and f_up = fp32(f (1 + 2^-20)), f = fp32(448 * rcp(m)), before rho is known.
The claim: for m and s normal, fp32(t * f_dn) < |q| < fp32(t * f_up) in
magnitude, whatever the hardware reciprocal's error within 1 ulp; hence where
the two e4m3 codes agree they are the code of q.  Emulated here in numpy fp32
arithmetic (one rounding per operation, as on the GPU), on products of bf16
values and rho spread over 2^-24 ... 2^24."""
import numpy as np
import pytest

from helpers import torch_e4m3fn

import workloads


def _slices(seed: int, n_groups: int, group: int = 16):
    rng = np.random.default_rng(seed)
    z = workloads.to_bf16_bits(rng.standard_normal((n_groups, group)).astype(np.float32))
    w = workloads.to_bf16_bits((1 + 0.1 * rng.standard_normal((n_groups, group))).astype(np.float32))
    zf = (z.astype(np.uint32) << 16).view(np.float32)
    wf = (w.astype(np.uint32) << 16).view(np.float32)
    t = zf * wf  # exact in fp32
    m = np.abs(t).max(axis=1).astype(np.float32)
    rho = np.exp2(rng.uniform(-24, 24, n_groups))
    return t, m, rho


def _bracket(t, m, ulps: int):
    """f_dn, f_up with the reciprocal of m taken `ulps` ulps off the correctly
    rounded one."""
    one = np.float32(1.0)
    rc = (one / m).astype(np.float32)
    rc = (rc.view(np.int32) + np.int32(ulps)).view(np.float32)
    f = (np.float32(448.0) * rc).astype(np.float32)
    f_dn = (f * np.float32(1.0 - 2.0 ** -20)).astype(np.float32)
    f_up = (f * np.float32(1.0 + 2.0 ** -20)).astype(np.float32)
    lo = (t * f_dn[:, None]).astype(np.float32)
    hi = (t * f_up[:, None]).astype(np.float32)
    return lo, hi


@pytest.mark.parametrize("ulps", [-1, 0, 1])
def test_bracket_encloses_the_quotient(ulps):
    t, m, rho = _slices(2024, 40000)
    rho448 = rho * (1.0 / 448.0)
    s = (m.astype(np.float64) * rho448).astype(np.float32)
    assert (s >= np.float32(2.0 ** -126)).all()  # normal scales, the bracket's premise
    q = t.astype(np.float64) * rho[:, None] / s.astype(np.float64)[:, None]
    lo, hi = _bracket(t, m, ulps)
    nz = t != 0
    a = np.abs(q)
    inside = (np.abs(lo.astype(np.float64)) < a) & (a < np.abs(hi.astype(np.float64)))
    assert inside[nz].all()
    # margin to the nearer end, relative: the analysis bounds it below by ~2^-20.8
    margin = np.minimum(a - np.abs(lo), np.abs(hi) - a)[nz] / a[nz]
    assert margin.min() > 2.0 ** -21


@pytest.mark.parametrize("ulps", [-1, 1])
def test_agreeing_codes_are_the_quotients_code(ulps):
    t, m, rho = _slices(77, 20000)
    s = (m.astype(np.float64) * (rho * (1.0 / 448.0))).astype(np.float32)
    q = t.astype(np.float64) * rho[:, None] / s.astype(np.float64)[:, None]
    lo, hi = _bracket(t, m, ulps)
    c_lo, c_hi = torch_e4m3fn(lo), torch_e4m3fn(hi)
    agree = c_lo == c_hi
    assert agree.mean() > 0.99
    # Where the bracket is closed, q lies more than 2^-21 from every e4m3
    # midpoint, so its fp32 rounding (torch converts through fp32) cannot
    # change its code.
    assert np.array_equal(c_lo[agree], torch_e4m3fn(q[agree]))


def test_amax_element_is_bracketed_near_448():
    """The slice's largest |t| has q = 448 / (1 + e): its bracket straddles or
    sits just below 448 and both codes are 448 (0x7E) or the bracket is open."""
    t, m, rho = _slices(5, 20000)
    idx = np.abs(t).argmax(axis=1)
    tm = t[np.arange(len(t)), idx][:, None]
    lo, hi = _bracket(tm, m, 0)
    c_lo, c_hi = torch_e4m3fn(np.abs(lo)), torch_e4m3fn(np.abs(hi))
    closed = c_lo == c_hi
    assert (c_lo[closed] == 0x7E).all()
