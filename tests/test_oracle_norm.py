"""Pins for the oracle's residual add + RMSNorm + FP8 quant.

Checks the oracle against a hand-worked example, closed forms of special rows,
invariants of the method (scale invariance, permutation equivariance, the
amax/448 rule, the format's error bound), torch's bf16 rounding of the
residual sum, and the unfused composition the fusion replaces."""
import math

import numpy as np
import pytest
import torch

import workloads
from helpers import TIE_CASES, bf16_to_f64, code_ulp_diff, e4m3_value, read_kv, torch_e4m3fn


def _bf16(vals):
    return np.array([int(np.float32(v).view(np.uint32) >> 16) for v in vals], np.uint16)


def _example():
    g = read_kv("norm_quant_worked_example.txt")
    f = lambda k: [float(v) for v in g[k]]
    h = lambda k: np.array([int(v, 16) for v in g[k]])
    return g, f, h


def test_worked_example(oracle):
    g, f, h = _example()
    x = _bf16(f("x"))[None, :]
    r = _bf16(f("residual"))[None, :]
    w = _bf16(f("weight"))
    eps = float(g["eps"][0])
    codes, scales, r_out = oracle.fused_add_rmsnorm_quant(
        x, r, w, eps, oracle.Q_STATIC, static_scale=float(g["static_scale"][0]))
    assert np.array_equal(bf16_to_f64(r_out[0]), np.array(f("residual_out")))
    assert np.array_equal(codes[0], h("static_codes"))
    codes, scales, _ = oracle.fused_add_rmsnorm_quant(x, r, w, eps, oracle.Q_PER_TOKEN)
    assert np.array_equal(codes[0], h("per_token_codes"))
    assert scales.view(np.uint32)[0] == h("per_token_scale_bits")[0]
    codes, scales, _ = oracle.fused_add_rmsnorm_quant(x, r, w, eps, oracle.Q_PER_GROUP, 2)
    assert np.array_equal(codes[0], h("per_group2_codes"))
    assert np.array_equal(scales.view(np.uint32)[0], h("per_group2_scale_bits"))


@pytest.mark.parametrize("c,eps", [(0.75, 1e-6), (-3.0, 1e-5), (0.015625, 1e-2), (2.5, 0.0)])
def test_constant_row_closed_form(oracle, c, eps):
    H = 256
    x = _bf16([c] * H)[None, :]
    w = _bf16([1.0] * H)
    y = c / math.sqrt(c * c + np.float64(np.float32(eps)))  # every element equals y
    codes, scales, _ = oracle.fused_add_rmsnorm_quant(x, None, w, eps, oracle.Q_PER_TOKEN)
    assert np.all(codes == (0xFE if c < 0 else 0x7E))
    assert scales[0] == np.float32(abs(y) / 448.0)
    s = 2.0 ** -5  # a power of two keeps y / s exact, so torch's float32 path is exact too
    codes, _, _ = oracle.fused_add_rmsnorm_quant(x, None, w, eps, oracle.Q_STATIC,
                                                 static_scale=s)
    assert np.all(codes == torch_e4m3fn([np.clip(y / s, -448, 448)])[0])


def test_single_element_row(oracle):
    for z, wv, eps in [(3.0, 0.5, 1e-6), (-0.125, 2.0, 1e-2)]:
        x = _bf16([z])[None, :]
        w = _bf16([wv])
        y = z / math.sqrt(z * z + np.float64(np.float32(eps))) * wv
        codes, scales, _ = oracle.fused_add_rmsnorm_quant(x, None, w, eps, oracle.Q_PER_TOKEN)
        assert scales[0] == np.float32(abs(y) / 448.0)
        assert codes[0, 0] == (0xFE if y < 0 else 0x7E)


def test_residual_sum_matches_torch(oracle):
    d = workloads.norm_inputs(64, 1024)
    # widen the exponent spread so that some sums are not exact in bf16
    d["residual"][:, ::7] = workloads.to_bf16_bits(
        bf16_to_f64(d["residual"][:, ::7]).astype(np.float32) * np.float32(300.0))
    _, _, r_out = oracle.fused_add_rmsnorm_quant(d["x"], d["residual"], d["weight"], 1e-6,
                                                 oracle.Q_PER_TOKEN)
    tx = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).float()
    tr = torch.from_numpy(d["residual"].view(np.int16)).view(torch.bfloat16).float()
    ref = (tx + tr).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(r_out, ref)


def test_norm_reads_the_rounded_sum(oracle):
    """The residual is updated in place and the norm normalizes that updated
    residual ([FUSION] section "RMSNorm + Quantization"): its input is
    z = bf16(x + r), not the exact sum.  So every row must give exactly the
    codes and scales of normalizing bf16(x + r), rounded here by torch, passed
    as x with no residual.  A residual column in three is scaled up so that
    most sums need rounding.  (The fused == unfused pins cannot see this
    reading: both compositions share it.)"""
    d = workloads.norm_inputs(64, 1024, salt=3)
    d["residual"][:, ::3] = workloads.to_bf16_bits(
        bf16_to_f64(d["residual"][:, ::3]).astype(np.float32) * np.float32(37.0))
    tx = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).float()
    tr = torch.from_numpy(d["residual"].view(np.int16)).view(torch.bfloat16).float()
    z = (tx + tr).to(torch.bfloat16)  # the float32 sum is exact here; one rounding to bf16
    assert np.count_nonzero(z.double().numpy() != (tx.double() + tr.double()).numpy()) > 1000
    z_bits = z.view(torch.int16).numpy().view(np.uint16)
    for mode, g in ((oracle.Q_PER_TOKEN, 0), (oracle.Q_PER_GROUP, 128)):
        fused = oracle.fused_add_rmsnorm_quant(d["x"], d["residual"].copy(), d["weight"], 1e-6,
                                               mode, g)
        plain = oracle.fused_add_rmsnorm_quant(z_bits, None, d["weight"], 1e-6, mode, g)
        assert np.array_equal(fused[0], plain[0])
        assert np.array_equal(fused[1].view(np.uint32), plain[1].view(np.uint32))


def test_no_residual_equals_zero_residual(oracle):
    d = workloads.norm_inputs(8, 512)
    zero = np.zeros_like(d["residual"])
    a = oracle.fused_add_rmsnorm_quant(d["x"], None, d["weight"], 1e-5, oracle.Q_PER_TOKEN)
    b = oracle.fused_add_rmsnorm_quant(d["x"], zero, d["weight"], 1e-5, oracle.Q_PER_TOKEN)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(b[2], d["x"])


@pytest.mark.parametrize("mode,g", [(2, 0), (3, 128), (3, 64)])
def test_scale_invariance(oracle, mode, g):
    """With eps = 0 RMSNorm ignores the row's scale: doubling x and residual
    (exact in bf16) leaves codes and scales unchanged."""
    d = workloads.norm_inputs(16, 1024)
    dbl = lambda a: workloads.to_bf16_bits(bf16_to_f64(a).astype(np.float32) * 2)
    a = oracle.fused_add_rmsnorm_quant(d["x"], d["residual"], d["weight"], 0.0, mode, g)
    b = oracle.fused_add_rmsnorm_quant(dbl(d["x"]), dbl(d["residual"]), d["weight"], 0.0,
                                       mode, g)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_permutation_equivariance(oracle):
    d = workloads.norm_inputs(8, 512)
    perm = np.random.default_rng(5).permutation(512)
    a = oracle.fused_add_rmsnorm_quant(d["x"], d["residual"], d["weight"], 1e-5,
                                       oracle.Q_PER_TOKEN)
    b = oracle.fused_add_rmsnorm_quant(np.ascontiguousarray(d["x"][:, perm]),
                                       np.ascontiguousarray(d["residual"][:, perm]),
                                       d["weight"][perm], 1e-5, oracle.Q_PER_TOKEN)
    assert np.array_equal(a[0][:, perm], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(a[2][:, perm], b[2])


@pytest.mark.parametrize("mode,g", [(2, 0), (3, 128), (3, 64)])
def test_amax_rule(oracle, mode, g):
    """Every slice with a non-zero amax has its largest code at exactly 448."""
    d = workloads.norm_inputs(32, 4096)
    codes, scales, _ = oracle.fused_add_rmsnorm_quant(d["x"], d["residual"], d["weight"],
                                                      1e-5, mode, g)
    mag = np.abs(oracle.e4m3fn_decode_array(codes))
    assert np.all(np.isfinite(mag)) and mag.max() <= 448.0
    per = mag.reshape(32, -1) if mode == 2 else mag.reshape(32, 4096 // g, g)
    assert np.all(per.max(axis=-1) == 448.0)
    assert np.all(scales > 0)


def test_quant_error_bound(oracle):
    """|decode(code) * s - y| stays within the format's half-spacing: 2^-4 |y|
    in the normal range, 2^-10 s in the subnormal range (plus bf16 rounding of
    the y reference, taken from the oracle's bf16-output path)."""
    d = workloads.norm_inputs(16, 1536, tag="mla")
    codes, scales, _ = oracle.fused_add_rmsnorm_quant(d["x"], None, d["weight"], 1e-6,
                                                      oracle.Q_PER_GROUP, 128)
    kv = d["x"][:, :512]
    y16, _, _ = oracle.dual_rmsnorm_quant(d["x"], d["weight"], 1e-6, kv, d["weight"][:512],
                                          1e-6, oracle.Q_NONE)
    y = bf16_to_f64(y16)
    s = np.repeat(scales.astype(np.float64), 128, axis=1)
    deq = oracle.e4m3fn_decode_array(codes) * s
    bound = 2.0 ** -4 * np.abs(y) + 2.0 ** -8 * np.abs(y) + 2.0 ** -10 * s
    assert np.all(np.abs(deq - y) <= bound)


@pytest.mark.parametrize("H,mode,g,eps", [(1024, 1, 0, 1e-6), (4096, 2, 0, 1e-5),
                                          (4096, 3, 128, 1e-5), (2048, 3, 64, 1e-6)])
def test_fused_equals_unfused(oracle, H, mode, g, eps):
    d = workloads.norm_inputs(64, H)
    a = oracle.fused_add_rmsnorm_quant(d["x"], d["residual"], d["weight"], eps, mode, g, 0.05)
    b = oracle.unfused_add_rmsnorm_quant(d["x"], d["residual"], d["weight"], eps, mode, g, 0.05)
    assert np.array_equal(a[2], b[2])
    diff = code_ulp_diff(a[0], b[0])
    assert diff.max() <= 1 and 0 < np.count_nonzero(diff) < diff.size // 4
    if mode != 1:
        assert np.allclose(a[1], b[1], rtol=2.0 ** -8, atol=0)


def test_strided_rows(oracle):
    d = workloads.norm_inputs(8, 1024)
    wide_x = np.zeros((8, 1536), np.uint16)
    wide_x[:, :1024] = d["x"]
    wide_r = np.zeros((8, 2048), np.uint16)
    wide_r[:, 512:1536] = d["residual"]
    a = oracle.fused_add_rmsnorm_quant(d["x"], d["residual"], d["weight"], 1e-6, 2)
    b = oracle.fused_add_rmsnorm_quant(wide_x[:, :1024], wide_r[:, 512:1536], d["weight"],
                                       1e-6, 2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2])


def test_zero_row_gives_zero_scale_and_codes(oracle):
    x = np.zeros((2, 128), np.uint16)
    w = _bf16([1.0] * 128)
    codes, scales, _ = oracle.fused_add_rmsnorm_quant(x, None, w, 1e-6, oracle.Q_PER_TOKEN)
    assert np.all(scales == 0) and np.all(codes == 0)


def test_argument_errors(oracle):
    d = workloads.norm_inputs(2, 1000)
    with pytest.raises(oracle.OracleError) as e:
        oracle.fused_add_rmsnorm_quant(d["x"], None, d["weight"], 1e-6, oracle.Q_PER_GROUP, 128)
    assert e.value.rc == oracle.EARG
    with pytest.raises(oracle.OracleError) as e:
        oracle.fused_add_rmsnorm_quant(d["x"], None, d["weight"], 1e-6, oracle.Q_STATIC,
                                       static_scale=0.0)
    assert e.value.rc == oracle.ECONTRACT
    with pytest.raises(oracle.OracleError):
        oracle.fused_add_rmsnorm_quant(d["x"], None, d["weight"], 1e-6, 7)
    out = oracle.fused_add_rmsnorm_quant(d["x"][:0], None, d["weight"], 1e-6, 2)
    assert out[0].shape == (0, 1000)


def tie_row(z0, w0, H=8):
    x = _bf16([z0] + [0.0] * (H - 1))[None, :]
    w = _bf16([w0] + [1.0] * (H - 1))
    return x, w


@pytest.mark.parametrize("s,m,z0,w0,eps,code,side", TIE_CASES)
def test_exact_tie_rounds_to_even(oracle, s, m, z0, w0, eps, code, side):
    from fractions import Fraction as F

    H = 8
    # the construction is exact in every step
    assert all(float(np.float32(v)) == v for v in (s, eps, z0, w0))
    assert F(z0) ** 2 / H + F(eps) == 1 and F(z0) * F(w0) / F(s) == F(m)
    # m is half-way between the expected code and a neighbour, and that code is even
    lo, hi = (code - 1, code) if e4m3_value(code) > m else (code, code + 1)
    assert F(e4m3_value(lo)) + F(e4m3_value(hi)) == 2 * F(m) and code % 2 == 0
    # the reciprocal form misses the midpoint on the recorded side
    assert (z0 * w0 * (1.0 / s) > m) == (side == "up") and z0 * w0 * (1.0 / s) != m
    x, w = tie_row(z0, w0, H)
    codes, _, _ = oracle.fused_add_rmsnorm_quant(x, None, w, eps, oracle.Q_STATIC,
                                                  static_scale=s)
    assert codes[0, 0] == code and not codes[0, 1:].any()


def test_non_finite_rows(oracle):
    """The stated readings for non-finite rows: a NaN makes rho NaN and every
    value NaN, whose amax is 0, so each dynamic scale of the row is 0 with +0
    codes, and a static scale codes every value as NaN; an infinity makes
    rho 0, so the static codes are +-0 (sign of z * w) except NaN at the
    infinity itself.  Ordinary rows in the same call are unaffected."""
    H = 16
    w = workloads.to_bf16_bits(np.linspace(0.5, 1.5, H).astype(np.float32))
    x = np.ones((3, H), np.float32)
    x[0, 3] = np.nan
    x[1, 4] = np.inf
    x[1, 5] = -2.0
    xb = workloads.to_bf16_bits(x)
    for mode, g in ((2, 0), (3, 8)):
        codes, scales, _ = oracle.fused_add_rmsnorm_quant(xb, None, w, 1e-6, mode, g)
        assert (scales[:2] == 0).all() and (codes[:2] == 0).all()
        assert (scales[2] > 0).all() and (codes[2] != 0).all()
    codes, _, _ = oracle.fused_add_rmsnorm_quant(xb, None, w, 1e-6, 1, 0, 0.05)
    assert ((codes[0] & 0x7F) == 0x7F).all()
    assert (codes[1, 4] & 0x7F) == 0x7F
    assert codes[1, 5] == 0x80
    assert (codes[1, np.r_[0:4, 6:H]] == 0x00).all()
    ref, _, _ = oracle.fused_add_rmsnorm_quant(xb[2:], None, w, 1e-6, 1, 0, 0.05)
    assert np.array_equal(codes[2], ref[0])


@pytest.mark.parametrize("factor", [2.0 ** -100, 2.0 ** -120, 2.0 ** 100])
@pytest.mark.parametrize("mode,g", [(2, 0), (3, 64)])
def test_scale_invariance_at_range_ends(oracle, factor, mode, g):
    """The same law far from 1: with eps = 0, x scaled by 2^-100, 2^-120 or
    2^100 (exact in bf16 for these rows, whose values stay normal) gives the
    codes and scales of x, so rows near the ends of the range have a fixed
    expected answer."""
    rng = np.random.default_rng(21)
    x = workloads.to_bf16_bits((rng.uniform(0.5, 2.0, (8, 256)) *
                                rng.choice([-1, 1], (8, 256))).astype(np.float32))
    w = workloads.to_bf16_bits((1 + 0.1 * rng.standard_normal(256)).astype(np.float32))
    scaled = bf16_to_f64(x) * factor
    xs = workloads.to_bf16_bits(scaled.astype(np.float32))
    assert np.array_equal(bf16_to_f64(xs), scaled)  # the scaling is exact
    a = oracle.fused_add_rmsnorm_quant(x, None, w, 0.0, mode, g)
    b = oracle.fused_add_rmsnorm_quant(xs, None, w, 0.0, mode, g)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
