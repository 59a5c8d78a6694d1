"""Pins of the oracle's next-row functions against what the pages and the
mathematics fix (not against the oracle itself):

- QK norm + RoPE ("Fusion torch.compile passes", section "QK Norm + RoPE"):
  per-head RMSNorm then rotation, checked through a one-hot closed form (it
  fixes the norm's sqrt(D) gain, the weight, the neox pairing and the
  frequency at once), norm preservation, the relative-position property, the
  split of qkv into q / k / v, the cache placement, and fused == unfused.
- Residual add + RMSNorm + padding (section "RMSNorm + Padding"): the
  hand-worked norm example, exact +0 padding, the residual update; with fp16
  elements the same example and a closed form against numpy's fp16 rounding.
- MLA RoPE + cache concat (the MLA split of section "MLA Dual RMSNorm" with
  the cache write of section "RoPE + KV-Cache Update"): position 0 is a pure
  copy into [kv_c | k_pe], a one-hot pins GPT-J pairing, strided q heads keep
  their nope part, padding tokens write nothing.
"""
import dataclasses
import math

import numpy as np
import pytest

import workloads
from helpers import bf16_to_f64, read_kv

SMALL_QK = dataclasses.replace(workloads.QKNORM, Hq=4, Hkv=2, D=64, num_blocks=8, block_size=4,
                               max_pos=512)


def bf(x):
    """float64 -> bf16 bits via numpy float32 then truncation-free torch rounding."""
    from helpers import f64_to_bf16_torch

    return f64_to_bf16_torch(np.asarray(x, dtype=np.float64))


def qk_call(oracle, cfg, d, **kw):
    return oracle.qk_norm_rope_kv_write(d["positions"], d["qkv"], d["q_w"], d["k_w"], cfg.eps,
                                        cfg.theta, cfg.max_pos, cfg.Hq, cfg.Hkv, cfg.D, **kw)


def test_qknorm_one_hot_closed_form(oracle):
    """A one-hot head e_i with unit weights and eps = 0 normalizes to sqrt(D) e_i;
    at position p the rotation puts sqrt(D) cos(p w_i) at i and sqrt(D)
    sin(p w_i) at i + D/2, w_i = theta^(-2i/D)."""
    cfg = SMALL_QK
    D = cfg.D
    T = 3
    qkv = np.zeros((T, (cfg.Hq + 2 * cfg.Hkv) * D), np.float64)
    pos = np.array([0, 5, 77], np.int64)
    idx = [1, 7, 20]
    for t in range(T):
        for h in range(cfg.Hq + cfg.Hkv):
            qkv[t, h * D + idx[t]] = 0.5 + h  # any non-zero amplitude
    ones = bf(np.ones(D))
    out, _, _ = oracle.qk_norm_rope_kv_write(pos, bf(qkv), ones, ones, 0.0, cfg.theta,
                                             cfg.max_pos, cfg.Hq, cfg.Hkv, D, write_k=True)
    got = bf16_to_f64(out)
    for t in range(T):
        ang = pos[t] * cfg.theta ** (-2.0 * idx[t] / D)
        want = np.zeros(D)
        want[idx[t]] = math.sqrt(D) * math.cos(ang)
        want[idx[t] + D // 2] = math.sqrt(D) * math.sin(ang)
        for h in range(cfg.Hq + cfg.Hkv):
            np.testing.assert_allclose(got[t, h * D:(h + 1) * D], want, rtol=2 ** -8, atol=1e-6)


def test_qknorm_weights_apply_per_head_dimension(oracle):
    """At position 0 (identity rotation) q heads are scaled by q_w and k heads
    by k_w, element by element; v is untouched."""
    cfg = SMALL_QK
    D = cfg.D
    d = workloads.qknorm_inputs(5, cfg)
    pos = np.zeros(5, np.int64)
    out, _, _ = oracle.qk_norm_rope_kv_write(pos, d["qkv"], d["q_w"], d["k_w"], cfg.eps,
                                             cfg.theta, cfg.max_pos, cfg.Hq, cfg.Hkv, D,
                                             write_k=True)
    x = bf16_to_f64(d["qkv"]).reshape(5, -1, D)
    got = bf16_to_f64(out).reshape(5, -1, D)
    rho = 1.0 / np.sqrt(np.mean(x ** 2, axis=2, keepdims=True) + np.float32(cfg.eps))
    w = np.concatenate([np.tile(bf16_to_f64(d["q_w"]), (cfg.Hq, 1)),
                        np.tile(bf16_to_f64(d["k_w"]), (cfg.Hkv, 1))])
    want = x[:, :cfg.Hq + cfg.Hkv] * rho[:, :cfg.Hq + cfg.Hkv] * w[None]
    np.testing.assert_allclose(got[:, :cfg.Hq + cfg.Hkv], want, rtol=2 ** -8, atol=1e-6)
    assert np.array_equal(out.reshape(5, -1, D)[:, cfg.Hq + cfg.Hkv:],
                          d["qkv"].reshape(5, -1, D)[:, cfg.Hq + cfg.Hkv:])


def test_qknorm_rotation_keeps_unit_rms(oracle):
    """With unit weights and eps = 0 every output head has mean square 1 at any
    position (RMSNorm gives 1, the rotation preserves pair norms)."""
    cfg = SMALL_QK
    d = workloads.qknorm_inputs(16, cfg)
    ones = bf(np.ones(cfg.D))
    out, _, _ = oracle.qk_norm_rope_kv_write(d["positions"], d["qkv"], ones, ones, 0.0,
                                             cfg.theta, cfg.max_pos, cfg.Hq, cfg.Hkv, cfg.D,
                                             write_k=True)
    heads = bf16_to_f64(out).reshape(16, -1, cfg.D)[:, :cfg.Hq + cfg.Hkv]
    np.testing.assert_allclose(np.mean(heads ** 2, axis=2), 1.0, rtol=2 ** -7)


def test_qknorm_relative_position(oracle):
    """<q at position m, k at position n> depends only on m - n (computed on the
    rounded outputs, within bf16 accuracy)."""
    cfg = dataclasses.replace(SMALL_QK, Hq=1, Hkv=1)
    d = workloads.qknorm_inputs(1, cfg)
    row = np.repeat(d["qkv"], 4, axis=0)
    pos = np.array([10, 3, 107, 100], np.int64)  # pairs (10, 3) and (107, 100): m - n = 7
    out, _, _ = oracle.qk_norm_rope_kv_write(pos, row, d["q_w"], d["k_w"], cfg.eps, cfg.theta,
                                             cfg.max_pos, 1, 1, cfg.D, write_k=True)
    o = bf16_to_f64(out).reshape(4, 3, cfg.D)
    a = np.dot(o[0, 0], o[1, 1])
    b = np.dot(o[2, 0], o[3, 1])
    assert abs(a - b) <= 0.02 * max(1.0, abs(a))


def test_qknorm_cache_write(oracle):
    """Rotated k lands at the token's slot (block slot // B, offset slot % B),
    v is bit-copied next to it, padding tokens and every other slot are left
    alone, and the cached k equals the k written back into qkv."""
    cfg = SMALL_QK
    T = 9
    d = workloads.qknorm_inputs(T, cfg)
    slots = d["slot_mapping"].copy()
    slots[[2, 6]] = -1
    out, kc, vc = qk_call(oracle, cfg, d, slot_mapping=slots, key_cache=d["key_cache"],
                          value_cache=d["value_cache"], write_k=True)
    D, Hq, Hkv = cfg.D, cfg.Hq, cfg.Hkv
    n = cfg.num_blocks * cfg.block_size
    k_back = out[:, Hq * D:(Hq + Hkv) * D].reshape(T, Hkv, D)
    v_in = d["qkv"][:, (Hq + Hkv) * D:].reshape(T, Hkv, D)
    kc2, vc2 = kc.reshape(n, Hkv, D), vc.reshape(n, Hkv, D)
    written = np.zeros(n, bool)
    for t in range(T):
        if slots[t] < 0:
            continue
        written[slots[t]] = True
        b, o = divmod(int(slots[t]), cfg.block_size)
        assert np.array_equal(kc[b, o], k_back[t])
        assert np.array_equal(vc[b, o], v_in[t])
    assert np.array_equal(kc2[~written], d["key_cache"].reshape(n, Hkv, D)[~written])
    assert np.array_equal(vc2[~written], d["value_cache"].reshape(n, Hkv, D)[~written])


def test_qknorm_without_k_writeback(oracle):
    """write_k = 0 leaves the k and v parts of qkv as they were."""
    cfg = SMALL_QK
    d = workloads.qknorm_inputs(4, cfg)
    out, _, _ = qk_call(oracle, cfg, d, slot_mapping=d["slot_mapping"],
                        key_cache=d["key_cache"], value_cache=d["value_cache"], write_k=False)
    q_cols = cfg.Hq * cfg.D
    assert np.array_equal(out[:, q_cols:], d["qkv"][:, q_cols:])
    assert not np.array_equal(out[:, :q_cols], d["qkv"][:, :q_cols])


@pytest.mark.parametrize("is_neox", [True, False])
def test_qknorm_fused_equals_unfused(oracle, is_neox):
    """The page's unfused sequence (bf16 q_norm / k_norm, then rotary) and the
    fused op differ only by that intermediate rounding: at most 2^-9 (|a| + |b|)
    for a rotated pair (a, b) of normalized values (|a|, |b| below ~4 here),
    plus the final bf16 rounding, so within 2^-6 absolute, 2^-7 relative."""
    cfg = SMALL_QK
    d = workloads.qknorm_inputs(12, cfg)
    kw = dict(slot_mapping=d["slot_mapping"], key_cache=d["key_cache"],
              value_cache=d["value_cache"], write_k=True, is_neox=is_neox)
    a, ka, va = qk_call(oracle, cfg, d, **kw)
    b, kb, vb = oracle.unfused_qk_norm_rope_kv_write(d["positions"], d["qkv"], d["q_w"],
                                                     d["k_w"], cfg.eps, cfg.theta, cfg.max_pos,
                                                     cfg.Hq, cfg.Hkv, cfg.D, **kw)
    np.testing.assert_allclose(bf16_to_f64(a), bf16_to_f64(b), rtol=2 ** -7, atol=2 ** -6)
    np.testing.assert_allclose(bf16_to_f64(ka), bf16_to_f64(kb), rtol=2 ** -7, atol=2 ** -6)
    assert np.mean(a == b) > 0.6  # most outputs are bit-identical despite the extra rounding
    assert np.array_equal(va, vb)


def test_qknorm_contract(oracle):
    cfg = SMALL_QK
    d = workloads.qknorm_inputs(4, cfg)
    bad = d["slot_mapping"].copy()
    bad[1] = bad[0]
    with pytest.raises(oracle.OracleError):
        qk_call(oracle, cfg, d, slot_mapping=bad, key_cache=d["key_cache"],
                value_cache=d["value_cache"])
    pos = d["positions"].copy()
    pos[0] = cfg.max_pos
    with pytest.raises(oracle.OracleError):
        oracle.qk_norm_rope_kv_write(pos, d["qkv"], d["q_w"], d["k_w"], cfg.eps, cfg.theta,
                                     cfg.max_pos, cfg.Hq, cfg.Hkv, cfg.D)


# ---- residual add + RMSNorm + padding -------------------------------------------

def test_pad_worked_example(oracle):
    """The hand-worked norm example (eps = 0, mean(z^2) = 1): y = z * w exactly,
    then 4 columns of +0 padding."""
    ex = read_kv("norm_quant_worked_example.txt")
    vals = lambda k: np.array([float(v) for v in ex[k]])
    x, r, w = bf(vals("x")), bf(vals("residual")), bf(vals("weight"))
    out, res = oracle.fused_add_rmsnorm_pad(x[None], r[None], w, 0.0, 8)
    assert np.array_equal(bf16_to_f64(res[0]), vals("residual_out"))
    assert list(bf16_to_f64(out[0, :4])) == [1.0, -0.75, 0.5, -0.328125]
    assert np.array_equal(out[0, 4:], np.zeros(4, np.uint16))


def test_pad_matches_norm_and_zero_fills(oracle):
    """The first H columns equal the bf16 RMSNorm of z = bf16(x + residual)
    (the residual update is bit-identical to the norm+quant op's); the pad is
    +0 bit patterns."""
    cfg = workloads.PAD
    d = workloads.pad_inputs(7, cfg)
    out, res = oracle.fused_add_rmsnorm_pad(d["x"], d["residual"], d["weight"], cfg.eps,
                                            cfg.H_pad)
    _, _, res2 = oracle.fused_add_rmsnorm_quant(d["x"], d["residual"], d["weight"], cfg.eps, 2)
    assert np.array_equal(res, res2)
    z = bf16_to_f64(res)
    rho = 1.0 / np.sqrt(np.mean(z ** 2, axis=1, keepdims=True) + np.float32(cfg.eps))
    want = z * rho * bf16_to_f64(d["weight"])[None]
    np.testing.assert_allclose(bf16_to_f64(out[:, :cfg.H]), want, rtol=2 ** -8, atol=1e-30)
    assert np.array_equal(out[:, cfg.H:], np.zeros((7, cfg.H_pad - cfg.H), np.uint16))


def test_pad_without_residual_and_no_padding(oracle):
    cfg = workloads.PAD
    d = workloads.pad_inputs(3, cfg)
    a, res = oracle.fused_add_rmsnorm_pad(d["x"], None, d["weight"], cfg.eps, cfg.H)
    assert res is None and a.shape == (3, cfg.H)
    b, _ = oracle.fused_add_rmsnorm_pad(d["x"], None, d["weight"], cfg.eps, cfg.H_pad)
    assert np.array_equal(a, b[:, :cfg.H])


def _f16(a):
    return np.asarray(a, np.float64).astype(np.float16).view(np.uint16)


def _f16_to_f64(h):
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float64)


def test_pad_f16_worked_example(oracle):
    """The worked example's values are exact in fp16 too, so the fp16 op gives
    the same y = z * w and residual."""
    ex = read_kv("norm_quant_worked_example.txt")
    vals = lambda k: np.array([float(v) for v in ex[k]])
    x, r, w = _f16(vals("x")), _f16(vals("residual")), _f16(vals("weight"))
    assert np.array_equal(_f16_to_f64(x), vals("x"))
    out, res = oracle.fused_add_rmsnorm_pad(x[None], r[None], w, 0.0, 8, dtype="f16")
    assert np.array_equal(_f16_to_f64(res[0]), vals("residual_out"))
    assert list(_f16_to_f64(out[0, :4])) == [1.0, -0.75, 0.5, -0.328125]
    assert np.array_equal(out[0, 4:], np.zeros(4, np.uint16))


def test_pad_f16_closed_form(oracle):
    """fp16 elements: the residual is numpy's one-rounding fp16 of x + residual,
    and each output is within half an fp16 unit of z * rho * w computed in
    double (the op rounds the exact value once); the pad is +0."""
    cfg = workloads.PAD_F16
    d = workloads.pad_inputs(9, cfg)
    out, res = oracle.fused_add_rmsnorm_pad(d["x"], d["residual"], d["weight"], cfg.eps,
                                            cfg.H_pad, dtype="f16")
    z = _f16_to_f64(d["x"]) + _f16_to_f64(d["residual"])
    assert np.array_equal(res, _f16(z))
    z = _f16_to_f64(res)
    rho = 1.0 / np.sqrt(np.mean(z ** 2, axis=1, keepdims=True) + np.float32(cfg.eps))
    want = z * rho * _f16_to_f64(d["weight"])[None]
    got = _f16_to_f64(out[:, :cfg.H])
    assert np.all(np.abs(got - want) <= 2.0 ** -11 * np.abs(want) + 2.0 ** -25)
    assert np.array_equal(out[:, cfg.H:], np.zeros((9, cfg.H_pad - cfg.H), np.uint16))
    # read as bf16 the same bits would give a different row: the type is honoured
    other, _ = oracle.fused_add_rmsnorm_pad(d["x"], d["residual"], d["weight"], cfg.eps,
                                            cfg.H_pad)
    assert not np.array_equal(other, out)


# ---- MLA RoPE + cache concat ------------------------------------------------------

SMALL_MLA = dataclasses.replace(workloads.MLA_ROPE, Hq=3, num_blocks=4, block_size=4,
                                max_pos=256)


def mla_call(oracle, cfg, d, pos=None, slots=None):
    return oracle.mla_rope_kv_write(
        d["positions"] if pos is None else pos, d["q"], d["k_pe"], d["kv_c"], cfg.theta,
        cfg.max_pos, d["slot_mapping"] if slots is None else slots, d["kv_cache"], cfg.Hq,
        cfg.rope_dim, q_head_stride=cfg.nope + cfg.rope_dim, q_pe_offset=cfg.nope,
        is_neox=cfg.is_neox)


def test_mla_position_zero_is_a_copy(oracle):
    """At position 0 the cache row is exactly [kv_c | k_pe] and q is unchanged."""
    cfg = SMALL_MLA
    T = 5
    d = workloads.mla_rope_inputs(T, cfg)
    q, cache = mla_call(oracle, cfg, d, pos=np.zeros(T, np.int64))
    assert np.array_equal(q, d["q"])
    flat = cache.reshape(-1, cfg.kv_lora + cfg.rope_dim)
    for t in range(T):
        assert np.array_equal(flat[d["slot_mapping"][t]], np.concatenate([d["kv_c"][t],
                                                                          d["k_pe"][t]]))


def test_mla_gptj_pairing_one_hot(oracle):
    """GPT-J pairing: a one-hot k_pe at element 2i rotates into elements 2i and
    2i + 1 as (cos, sin) of p * theta^(-2i/rope_dim); q_pe heads likewise, and
    the nope part of each q head is untouched."""
    cfg = SMALL_MLA
    T, i, p = 2, 3, 41
    d = workloads.mla_rope_inputs(T, cfg)
    k_pe = np.zeros((T, cfg.rope_dim))
    k_pe[:, 2 * i] = 1.0
    d["k_pe"] = bf(k_pe)
    q = bf16_to_f64(d["q"]).reshape(T, cfg.Hq, -1)
    q[:, :, cfg.nope:] = 0.0
    q[:, :, cfg.nope + 2 * i] = 2.0
    d["q"] = bf(q.reshape(T, -1))
    q_out, cache = mla_call(oracle, cfg, d, pos=np.full(T, p, np.int64))
    ang = p * cfg.theta ** (-2.0 * i / cfg.rope_dim)
    want = np.zeros(cfg.rope_dim)
    want[2 * i], want[2 * i + 1] = math.cos(ang), math.sin(ang)
    flat = cache.reshape(-1, cfg.kv_lora + cfg.rope_dim)
    for t in range(T):
        np.testing.assert_allclose(bf16_to_f64(flat[d["slot_mapping"][t], cfg.kv_lora:]), want,
                                   atol=2 ** -8)
    qo = bf16_to_f64(q_out).reshape(T, cfg.Hq, -1)
    np.testing.assert_allclose(qo[:, :, cfg.nope:], 2.0 * np.broadcast_to(want, qo[:, :, cfg.nope:].shape),
                               atol=2 ** -7)
    assert np.array_equal(q_out.reshape(T, cfg.Hq, -1)[:, :, :cfg.nope],
                          d["q"].reshape(T, cfg.Hq, -1)[:, :, :cfg.nope])


def test_mla_padding_and_untouched_slots(oracle):
    cfg = SMALL_MLA
    T = 6
    d = workloads.mla_rope_inputs(T, cfg)
    slots = d["slot_mapping"].copy()
    slots[[1, 4]] = -1
    _, cache = mla_call(oracle, cfg, d, slots=slots)
    flat, flat0 = cache.reshape(-1, cfg.kv_lora + cfg.rope_dim), d["kv_cache"].reshape(
        -1, cfg.kv_lora + cfg.rope_dim)
    written = np.zeros(flat.shape[0], bool)
    written[slots[slots >= 0]] = True
    assert np.array_equal(flat[~written], flat0[~written])
    assert np.array_equal(flat[slots[slots >= 0], :cfg.kv_lora], d["kv_c"][slots >= 0])


def test_mla_k_pe_matches_single_head_rope(oracle):
    """The rotated k_pe in the cache equals rope_kv_write's key-cache entry for a
    single kv head of rope_dim (same pairing and frequencies)."""
    cfg = SMALL_MLA
    T = 4
    d = workloads.mla_rope_inputs(T, cfg)
    _, cache = mla_call(oracle, cfg, d)
    n = cfg.num_blocks * cfg.block_size
    zeros = np.zeros((n // cfg.block_size, cfg.block_size, 1, cfg.rope_dim), np.uint16)
    _, kc, _ = oracle.rope_kv_write(d["positions"], d["k_pe"].reshape(T, 1, -1),
                                    d["k_pe"].reshape(T, 1, -1), d["k_pe"].reshape(T, 1, -1),
                                    cfg.theta, cfg.max_pos, d["slot_mapping"], zeros, zeros, 1, 1,
                                    cfg.rope_dim, is_neox=cfg.is_neox)
    flat = cache.reshape(n, -1)
    assert np.array_equal(flat[d["slot_mapping"], cfg.kv_lora:],
                          kc.reshape(n, -1)[d["slot_mapping"]])


@pytest.mark.parametrize("factor", [2.0 ** -110, 2.0 ** 100])
def test_qknorm_scale_invariance_at_range_ends(oracle, factor):
    """With eps = 0 the per-head norm ignores a power-of-two scale of q and k
    (exact in bf16 for these values), so heads near the ends of the range have
    the outputs of ordinary ones."""
    import dataclasses

    cfg = dataclasses.replace(workloads.QKNORM, Hq=4, Hkv=2, eps=0.0)
    d = workloads.qknorm_inputs(5, cfg, with_cache=False)
    rng = np.random.default_rng(22)
    n = (cfg.Hq + cfg.Hkv) * cfg.D
    vals = rng.uniform(0.5, 2.0, (5, n)) * rng.choice([-1, 1], (5, n))
    base = d["qkv"].copy()
    base[:, :n] = workloads.to_bf16_bits(vals.astype(np.float32))
    scaled = base.copy()
    scaled[:, :n] = workloads.to_bf16_bits((vals * factor).astype(np.float32))
    assert np.array_equal(bf16_to_f64(scaled[:, :n]), bf16_to_f64(base[:, :n]) * factor)
    args = (d["q_w"], d["k_w"], 0.0, cfg.theta, cfg.max_pos, cfg.Hq, cfg.Hkv, cfg.D)
    a, _, _ = oracle.qk_norm_rope_kv_write(d["positions"], base, *args, write_k=True)
    b, _, _ = oracle.qk_norm_rope_kv_write(d["positions"], scaled, *args, write_k=True)
    assert np.array_equal(a[:, :n], b[:, :n])
