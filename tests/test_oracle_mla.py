"""Pins for the oracle's MLA dual RMSNorm (+ FP8 quant of the q latent).

The fused op must equal two independent single-row norms (the unfused
listings), its quantized q side must equal the residual-free case of the norm +
quant op, and its bf16 outputs must follow closed forms of special rows."""
import math

import numpy as np
import pytest

import workloads
from helpers import bf16_to_f64


def _bf16(vals):
    return workloads.to_bf16_bits(np.asarray(vals, np.float32))


@pytest.mark.parametrize("mode,g", [(0, 0), (2, 0), (3, 128), (3, 64)])
def test_fused_equals_unfused(oracle, mode, g):
    d = workloads.mla_inputs(32)
    a = oracle.dual_rmsnorm_quant(d["q"], d["q_w"], 1e-6, d["kv"], d["kv_w"], 1e-5, mode, g)
    b = oracle.unfused_dual_rmsnorm_quant(d["q"], d["q_w"], 1e-6, d["kv"], d["kv_w"], 1e-5,
                                          mode, g)
    for x, y in zip(a, b):
        assert (x is None and y is None) or np.array_equal(x, y)


@pytest.mark.parametrize("mode,g", [(2, 0), (3, 128)])
def test_q_side_equals_norm_quant(oracle, mode, g):
    d = workloads.mla_inputs(16)
    q_codes, q_scales, _ = oracle.dual_rmsnorm_quant(d["q"], d["q_w"], 1e-6, d["kv"], d["kv_w"],
                                                     1e-6, mode, g)
    codes, scales, _ = oracle.fused_add_rmsnorm_quant(d["q"], None, d["q_w"], 1e-6, mode, g)
    assert np.array_equal(q_codes, codes) and np.array_equal(q_scales, scales)


def test_sides_are_independent(oracle):
    d = workloads.mla_inputs(8)
    a = oracle.dual_rmsnorm_quant(d["q"], d["q_w"], 1e-6, d["kv"], d["kv_w"], 1e-6, 3, 128)
    kv2 = np.ascontiguousarray(d["kv"][::-1])
    b = oracle.dual_rmsnorm_quant(d["q"], d["q_w"], 1e-6, kv2, d["kv_w"], 1e-2, 3, 128)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(a[2][::-1], oracle.dual_rmsnorm_quant(
        d["q"], d["q_w"], 1e-6, kv2, d["kv_w"], 1e-6, 3, 128)[2])


@pytest.mark.parametrize("c,eps", [(0.5, 1e-6), (-2.0, 1e-2)])
def test_constant_row_closed_form(oracle, c, eps):
    w = _bf16([1.0, 0.5, -0.75, 2.0] * 128)
    kv = _bf16([[c] * 512])
    q = _bf16([[1.0] * 512])
    _, _, kv_out = oracle.dual_rmsnorm_quant(q, w, 1e-6, kv, w, eps, 0)
    y = c / math.sqrt(c * c + float(np.float32(eps))) * bf16_to_f64(w)
    expect = workloads.to_bf16_bits(y.astype(np.float32))  # y*w with w in {1, .5, -.75, 2}
    assert np.array_equal(kv_out[0], expect)


@pytest.mark.parametrize("cq,eps_q,ckv,eps_kv", [(0.1, 1e-2, 0.25, 1e-6), (0.3, 1e-6, 0.1, 3e-2)])
def test_each_side_uses_its_own_weight_and_eps(oracle, cq, eps_q, ckv, eps_kv):
    """Constant rows whose epsilons matter (c^2 and eps of the same order), with
    different weights and epsilons on the two sides: a side that took the
    other's weight or eps would be off by far more than a bf16 step."""
    wq = _bf16([1.0, 0.5, -0.75, 2.0] * 384)
    wkv = _bf16([1.5, -0.25, 0.75, 1.0] * 128)
    q = _bf16([[cq] * 1536])
    kv = _bf16([[ckv] * 512])
    q_out, _, kv_out = oracle.dual_rmsnorm_quant(q, wq, eps_q, kv, wkv, eps_kv, 0)
    for out, c, eps, w in ((q_out, cq, eps_q, wq), (kv_out, ckv, eps_kv, wkv)):
        cb = float(bf16_to_f64(_bf16([c]))[0])  # the row value as stored
        y = cb / math.sqrt(cb * cb + float(np.float32(eps))) * bf16_to_f64(w)
        got = bf16_to_f64(out[0])
        assert np.allclose(got, y, rtol=2 ** -8, atol=0)
        # the other side's eps or weight would not do
        other = cb / math.sqrt(cb * cb + float(np.float32(eps_kv if eps == eps_q else eps_q)))
        assert not np.allclose(got[:4], other * bf16_to_f64(w)[:4], rtol=2 ** -6)


def test_unit_rms_with_zero_eps(oracle):
    d = workloads.mla_inputs(4)
    w = _bf16([1.0] * 512)
    _, _, kv_out = oracle.dual_rmsnorm_quant(d["q"], d["q_w"], 0.0, d["kv"], w, 0.0, 0)
    ms = (bf16_to_f64(kv_out) ** 2).mean(axis=1)
    assert np.allclose(ms, 1.0, rtol=2 ** -7)


def test_strided_split_views(oracle):
    """q and kv may be column slices of one projected row block."""
    d = workloads.mla_inputs(8)
    proj = np.zeros((8, 1536 + 576), np.uint16)
    proj[:, :1536] = d["q"]
    proj[:, 1536:2048] = d["kv"]
    a = oracle.dual_rmsnorm_quant(d["q"], d["q_w"], 1e-6, d["kv"], d["kv_w"], 1e-6, 3, 128)
    b = oracle.dual_rmsnorm_quant(proj[:, :1536], d["q_w"], 1e-6, proj[:, 1536:2048], d["kv_w"],
                                  1e-6, 3, 128)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_argument_errors(oracle):
    d = workloads.mla_inputs(2)
    with pytest.raises(oracle.OracleError):  # static mode is not offered for the q latent
        oracle.dual_rmsnorm_quant(d["q"], d["q_w"], 1e-6, d["kv"], d["kv_w"], 1e-6, 1)
    with pytest.raises(oracle.OracleError):
        oracle.dual_rmsnorm_quant(d["q"], d["q_w"], 1e-6, d["kv"], d["kv_w"], 1e-6, 3, 100)
