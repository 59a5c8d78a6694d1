"""Pins for the oracle's SiLU-and-Mul + FP8 quant.

SiLU is checked on every finite bf16 gate value against the identity
sigmoid(x) = (1 + tanh(x/2)) / 2 evaluated with numpy; the multiplication by
the up half, the half order, the amax/448 group rule and the unfused
composition are pinned separately."""
import numpy as np
import pytest

import workloads
from helpers import bf16_to_f64, code_ulp_diff, torch_e4m3fn

ONE = np.uint16(0x3F80)  # bf16 1.0


def _all_finite_bf16() -> np.ndarray:
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return h[(h & 0x7F80) != 0x7F80]


def _gate_up(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.concatenate([gate, up], axis=1))


def test_silu_on_every_bf16_gate(oracle):
    g = _all_finite_bf16()
    n = g.size - g.size % 128
    g = g[:n].reshape(-1, 128)
    inp = _gate_up(g, np.full_like(g, ONE))
    s = 2.0 ** -6  # power of two: a / s stays exact
    codes, _ = oracle.silu_mul_quant(inp, oracle.Q_STATIC, static_scale=s)
    x = bf16_to_f64(g)
    silu = x * 0.5 * (1.0 + np.tanh(0.5 * x))
    ref = torch_e4m3fn(np.clip(silu / s, -448.0, 448.0))
    assert code_ulp_diff(codes, ref).max() == 0


def test_up_scaling_and_half_order(oracle):
    """silu(g) * 2u quantized with scale s equals silu(g) * u with scale s/2,
    and swapping the halves changes the result."""
    d = workloads.silu_inputs(4, 1024)
    g, u = d["inp"][:, :1024], d["inp"][:, 1024:]
    u2 = workloads.to_bf16_bits(bf16_to_f64(u).astype(np.float32) * 2)
    a, _ = oracle.silu_mul_quant(_gate_up(g, u2), oracle.Q_STATIC, static_scale=0.25)
    b, _ = oracle.silu_mul_quant(_gate_up(g, u), oracle.Q_STATIC, static_scale=0.125)
    assert np.array_equal(a, b)
    c, _ = oracle.silu_mul_quant(_gate_up(u, g), oracle.Q_STATIC, static_scale=0.125)
    assert np.count_nonzero(code_ulp_diff(b, c) > 1) > b.size // 2


def test_silu_zero(oracle):
    inp = np.zeros((1, 256), np.uint16)
    inp[0, 128:] = ONE
    codes, scales = oracle.silu_mul_quant(inp, oracle.Q_PER_GROUP, 128)
    assert np.all(codes == 0) and scales[0, 0] == 0


@pytest.mark.parametrize("g", [128, 64])
def test_group_scales(oracle, g):
    d = workloads.silu_inputs(8, 2048)
    codes, scales = oracle.silu_mul_quant(d["inp"], oracle.Q_PER_GROUP, g)
    x = bf16_to_f64(d["inp"][:, :2048])
    u = bf16_to_f64(d["inp"][:, 2048:])
    a = x * 0.5 * (1.0 + np.tanh(0.5 * x)) * u
    amax = np.abs(a).reshape(8, 2048 // g, g).max(axis=-1)
    ref = (amax / 448.0).astype(np.float32)
    assert np.all(np.abs(scales.view(np.int32) - ref.view(np.int32)) <= 1)  # within 1 fp32 ulp
    mag = np.abs(oracle.e4m3fn_decode_array(codes)).reshape(8, 2048 // g, g)
    assert np.all(mag.max(axis=-1) == 448.0)


@pytest.mark.parametrize("mode,g", [(1, 0), (3, 128), (3, 64)])
def test_fused_equals_unfused(oracle, mode, g):
    d = workloads.silu_inputs(32, 14336 // 4)
    a = oracle.silu_mul_quant(d["inp"], mode, g, 0.05)
    b = oracle.unfused_silu_mul_quant(d["inp"], mode, g, 0.05)
    diff = code_ulp_diff(a[0], b[0])
    assert diff.max() <= 1 and 0 < np.count_nonzero(diff) < diff.size // 4
    if mode == 3:
        assert np.allclose(a[1], b[1], rtol=2.0 ** -8, atol=0)


def test_argument_errors(oracle):
    d = workloads.silu_inputs(2, 200)
    with pytest.raises(oracle.OracleError):
        oracle.silu_mul_quant(d["inp"], oracle.Q_PER_GROUP, 128)
    with pytest.raises(oracle.OracleError):
        oracle.silu_mul_quant(d["inp"], oracle.Q_STATIC, static_scale=-1.0)


def test_non_finite_activations(oracle):
    """The stated readings for SiLU: a NaN activation codes as NaN and is left
    out of its group's amax; an infinite one makes the group's scale infinite
    (its finite values then code as +-0); a group of zero products gets scale 0
    and +0 codes, also for -0.0; a static scale saturates an infinity to 448."""
    G, I = 8, 32
    g = np.full((1, I), 1.0, np.float32)
    u = np.full((1, I), 1.0, np.float32)
    g[0, 2] = np.nan
    u[0, 9] = np.inf
    g[0, 16:24] = -0.0
    inp = np.concatenate([workloads.to_bf16_bits(g), workloads.to_bf16_bits(u)], axis=1)
    codes, scales = oracle.silu_mul_quant(inp, 3, G)
    silu1 = 1.0 / (1.0 + np.exp(-1.0))
    assert (codes[0, 2] & 0x7F) == 0x7F
    assert scales[0, 0] == np.float32(silu1 / 448.0)
    assert np.isinf(scales[0, 1]) and (codes[0, 8:16][np.arange(8) != 1] == 0).all()
    assert (codes[0, 9] & 0x7F) == 0x7F
    assert scales[0, 2] == 0 and (codes[0, 16:24] == 0).all()
    assert (codes[0, 24:32] == 0x7E).all()
    static, _ = oracle.silu_mul_quant(inp, 1, 0, 0.05)
    assert static[0, 9] == 0x7E and (static[0, 2] & 0x7F) == 0x7F


def test_products_beyond_fp32(oracle):
    """Per-group SiLU where silu(g) * u exceeds the fp32 range: scaling every u
    by 2^120 (exact in bf16 and in double) leaves every code unchanged and
    scales every group scale by exactly 2^120, as long as the scale itself
    stays finite in fp32; a group whose amax / 448 exceeds fp32 gets an
    infinite scale and codes +-0 (finite / inf)."""
    rng = np.random.default_rng(21)
    G, I = 128, 512
    g = (2.0 * rng.standard_normal((4, I))).astype(np.float32)
    u = rng.standard_normal((4, I)).astype(np.float32)
    g[:, :G] += 100.0  # silu(g) = g to double precision: products of a few hundred
    base = np.concatenate([workloads.to_bf16_bits(g), workloads.to_bf16_bits(u)], axis=1)
    big = np.concatenate([workloads.to_bf16_bits(g),
                          workloads.to_bf16_bits(u * np.float32(2.0 ** 120))], axis=1)
    c0, s0 = oracle.silu_mul_quant(base, 3, G)
    c1, s1 = oracle.silu_mul_quant(big, 3, G)
    assert np.abs(bf16_to_f64(big[:, I:]) * bf16_to_f64(big[:, :I])).max() > 3.5e38
    assert np.array_equal(c0, c1)
    assert np.array_equal(s1.astype(np.float64), s0.astype(np.float64) * 2.0 ** 120)
    assert np.isfinite(s1).all()
    huge = big.copy()
    huge[0, :G] = workloads.to_bf16_bits(np.full(G, 3e38, np.float32))
    huge[0, I:I + G] = workloads.to_bf16_bits(np.full(G, 3e38, np.float32))
    c2, s2 = oracle.silu_mul_quant(huge, 3, G)
    assert np.isinf(s2[0, 0]) and (c2[0, :G] == 0).all()
    assert np.array_equal(c2[1:], c1[1:]) and np.array_equal(c2[0, G:], c1[0, G:])
