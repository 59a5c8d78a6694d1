"""Pins for the oracle's RoPE + paged KV-cache write.

Rotation: identity at position 0; one-hot inputs expose the pairing (neox
partner i + D/2, GPT-J partner i + 1), the frequency of pair 0 (one radian per
position) and the geometric progression of the others; pair norms are kept;
q.k after rotation depends only on the position difference.  Cache write:
the PagedAttention block-table example, brute force over every injective
slot assignment on a tiny cache, sentinel preservation and the contract
errors.  The fp16 element type: identity at position 0, one-hot values equal
to numpy's fp16 rounding of cos and sin, and agreement with the bf16 path on
inputs that both types hold exactly."""
import itertools
import math

import numpy as np
import pytest

import workloads
from helpers import bf16_to_f64, read_kv

THETA = 500000.0


def _bf16(a):
    return workloads.to_bf16_bits(np.asarray(a, np.float32))


def _run(oracle, positions, q, k, v, slots, kc, vc, Hq, Hkv, D, theta=THETA, max_pos=1 << 20,
         rot_dim=None, is_neox=True, dtype="bf16"):
    return oracle.rope_kv_write(np.asarray(positions, np.int64), q, k, v, theta, max_pos,
                                np.asarray(slots, np.int64), kc, vc, Hq, Hkv, D, rot_dim, is_neox,
                                dtype)


def _empty_cache(num_blocks, block_size, Hkv, D, fill=0x7E7E):
    return np.full((num_blocks, block_size, Hkv, D), fill, np.uint16)


def test_position_zero_is_identity(oracle):
    d = workloads.rope_inputs(8, with_cache=False)
    kc = _empty_cache(4096, 16, 8, 128)
    q_out, kc2, vc2 = _run(oracle, np.zeros(8), d["q"], d["k"], d["v"], d["slot_mapping"], kc,
                           kc.copy(), 32, 8, 128)
    assert np.array_equal(q_out, d["q"])
    s = d["slot_mapping"]
    assert np.array_equal(kc2.reshape(-1, 8, 128)[s], d["k"])
    assert np.array_equal(vc2.reshape(-1, 8, 128)[s], d["v"])


@pytest.mark.parametrize("is_neox", [True, False])
def test_one_hot_pairing_and_first_frequency(oracle, is_neox):
    D = 128
    for i in (0, 5, 63):
        q = np.zeros((1, 1, D), np.uint16)
        q[0, 0, (i if is_neox else 2 * i)] = 0x3F80
        pos = 3
        q_out, _, _ = _run(oracle, [pos], q, q[:, :, :].copy(), q.copy(), [-1],
                           _empty_cache(1, 1, 1, D), _empty_cache(1, 1, 1, D), 1, 1, D,
                           is_neox=is_neox)
        o = bf16_to_f64(q_out[0, 0])
        a, b = (i, i + D // 2) if is_neox else (2 * i, 2 * i + 1)
        nz = set(np.flatnonzero(o))
        assert nz <= {a, b}
        if i == 0:  # pair 0 turns one radian per position
            assert q_out[0, 0, a] == _bf16([math.cos(pos)])[0]
            assert q_out[0, 0, b] == _bf16([math.sin(pos)])[0]
        assert abs(math.hypot(o[a], o[b]) - 1.0) < 2 ** -7


def test_frequencies_form_a_geometric_progression(oracle):
    """Angles recovered from one-hot outputs at position 1 shrink by
    theta^(2/D) from one pair to the next."""
    D = 16
    theta = 50.0
    q = np.zeros((1, D // 2, D), np.uint16)
    for i in range(D // 2):
        q[0, i, i] = 0x3F80
    q_out, _, _ = _run(oracle, [1], q, q[:, :1].copy(), q[:, :1].copy(), [-1],
                       _empty_cache(1, 1, 1, D), _empty_cache(1, 1, 1, D), D // 2, 1, D,
                       theta=theta)
    o = bf16_to_f64(q_out[0])
    ang = np.array([math.atan2(o[i, i + D // 2], o[i, i]) for i in range(D // 2)])
    assert abs(ang[0] - 1.0) < 2 ** -7
    ratios = ang[:-1] / ang[1:]
    assert np.allclose(ratios, theta ** (2.0 / D), rtol=2e-2)


def test_relative_position_property(oracle):
    """<rope(q, m), rope(k, n)> depends only on m - n."""
    D = 128
    d = workloads.rope_inputs(1, with_cache=False)
    q, k = d["q"][:, :1], d["k"][:, :1]

    def dot(m, n):
        qo, _, _ = _run(oracle, [m], q, k, k, [-1], _empty_cache(1, 1, 1, D),
                        _empty_cache(1, 1, 1, D), 1, 1, D)
        ko, _, _ = _run(oracle, [n], k, k, k, [-1], _empty_cache(1, 1, 1, D),
                        _empty_cache(1, 1, 1, D), 1, 1, D)
        return float(np.dot(bf16_to_f64(qo[0, 0]), bf16_to_f64(ko[0, 0])))

    base = dot(10, 3)
    for m, n in [(107, 100), (5007, 5000), (7, 0)]:
        assert abs(dot(m, n) - base) < 0.05 * (1 + abs(base))
    assert abs(dot(10, 9) - base) > 0.05 * (1 + abs(base))


def test_partial_rotary_passes_tail_through(oracle):
    d = workloads.rope_inputs(4, with_cache=False)
    q_out, _, _ = _run(oracle, d["positions"], d["q"], d["k"], d["v"], [-1] * 4,
                       _empty_cache(1, 1, 8, 128), _empty_cache(1, 1, 8, 128), 32, 8, 128,
                       rot_dim=64)
    assert np.array_equal(q_out[..., 64:], d["q"][..., 64:])
    assert not np.array_equal(q_out[..., :64], d["q"][..., :64])


def test_block_table_example(oracle):
    """The PagedAttention diagram: tokens land in block_table[t // B] at
    offset t % B; nothing else in the cache changes."""
    g = read_kv("paged_block_table.txt")
    B, nb = int(g["block_size"][0]), int(g["num_blocks"][0])
    slots_a = np.array([int(s) for s in g["slots_A"]])
    table_a = [int(b) for b in g["table_A"]]
    assert [table_a[t // B] * B + t % B for t in range(int(g["tokens_A"][0]))] == list(slots_a)
    slots_b = np.array([int(s) for s in g["slots_B"]])
    D, Hkv = 8, 1
    kc0 = _empty_cache(nb, B, Hkv, D)
    for slots in (slots_a, slots_b):
        T = slots.size
        k = _bf16(np.arange(T * D).reshape(T, 1, D) + 1.0)
        v = _bf16(-np.arange(T * D).reshape(T, 1, D) - 1.0)
        q = np.zeros((T, 1, D), np.uint16)
        _, kc, vc = _run(oracle, np.zeros(T), q, k, v, slots, kc0, kc0.copy(), 1, Hkv, D)
        for t, s in enumerate(slots):
            assert np.array_equal(kc[s // B, s % B], k[t]) and np.array_equal(vc[s // B, s % B], v[t])
        untouched = np.ones(nb * B, bool)
        untouched[slots] = False
        assert np.all(kc.reshape(nb * B, -1)[untouched] == 0x7E7E)
        assert np.all(vc.reshape(nb * B, -1)[untouched] == 0x7E7E)


def test_brute_force_tiny_cache(oracle):
    """2 blocks x 2 slots, 3 tokens: every injective assignment of slots (with
    -1 for padding) writes exactly the assigned slots with that token's rotated
    k (taken from the unfused path) and v."""
    D, Hkv, B, nb = 4, 1, 2, 2
    d = workloads.rope_inputs(3, workloads.RopeCfg("tiny", Hq=1, Hkv=1, D=D, rot_dim=D,
                                                   max_pos=64, num_blocks=nb, block_size=B),
                              with_cache=False)
    kc0 = _empty_cache(nb, B, Hkv, D)
    choices = [-1, 0, 1, 2, 3]
    n = 0
    for slots in itertools.product(choices, repeat=3):
        used = [s for s in slots if s >= 0]
        if len(used) != len(set(used)):
            continue
        n += 1
        _, kc, vc = _run(oracle, d["positions"], d["q"], d["k"], d["v"], slots, kc0, kc0.copy(),
                         1, Hkv, D, max_pos=64)
        _, k_rot, _, _ = oracle.unfused_rope_kv_write(
            d["positions"], d["q"], d["k"], d["v"], THETA, 64, np.full(3, -1), kc0, kc0, 1, Hkv, D)
        exp_k = kc0.copy()
        exp_v = kc0.copy()
        for t, s in enumerate(slots):
            if s >= 0:
                exp_k[s // B, s % B] = k_rot[t]
                exp_v[s // B, s % B] = d["v"][t]
        assert np.array_equal(kc, exp_k) and np.array_equal(vc, exp_v), slots
    assert n == 1 + 3 * 4 + 3 * 4 * 3 + 4 * 3 * 2  # 0, 1, 2 or 3 tokens placed


def test_fused_equals_unfused(oracle):
    d = workloads.rope_inputs(64)
    a = _run(oracle, d["positions"], d["q"], d["k"], d["v"], d["slot_mapping"], d["key_cache"],
             d["value_cache"], 32, 8, 128, max_pos=8192)
    b = oracle.unfused_rope_kv_write(d["positions"], d["q"], d["k"], d["v"], THETA, 8192,
                                     d["slot_mapping"], d["key_cache"], d["value_cache"], 32, 8,
                                     128)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1], b[2]) and np.array_equal(a[2], b[3])


def test_contract_errors(oracle):
    d = workloads.rope_inputs(4, with_cache=False)
    kc = _empty_cache(4096, 16, 8, 128)
    args = (d["q"], d["k"], d["v"])
    for pos, slots in [([0, 1, 2, 8192], d["slot_mapping"]),  # position past the table
                       ([0, 1, 2, -1], d["slot_mapping"]),  # negative position
                       (d["positions"], [5, 6, 5, 7]),  # duplicate slot
                       (d["positions"], [0, 1, 2, 65536])]:  # slot past the cache
        with pytest.raises(oracle.OracleError) as e:
            _run(oracle, pos, *args, slots, kc, kc, 32, 8, 128, max_pos=8192)
        assert e.value.rc == oracle.ECONTRACT
    with pytest.raises(oracle.OracleError) as e:
        _run(oracle, d["positions"], *args, d["slot_mapping"], kc, kc, 32, 8, 128, rot_dim=127)
    assert e.value.rc == oracle.EARG
    _run(oracle, d["positions"], *args, [-1, -1, 3, 4], kc, kc, 32, 8, 128, max_pos=8192)


# ---- fp16 elements ---------------------------------------------------------------

def _f16(a):
    return np.asarray(a, np.float64).astype(np.float16).view(np.uint16)


def _f16_to_f64(h):
    return np.asarray(h, np.uint16).view(np.float16).astype(np.float64)


def test_f16_position_zero_is_identity(oracle):
    rng = np.random.default_rng(5)
    q, k, v = (_f16(rng.standard_normal((8, H, 64))) for H in (4, 2, 2))
    kc = _empty_cache(8, 4, 2, 64)
    slots = rng.permutation(32)[:8]
    q_out, kc2, vc2 = _run(oracle, np.zeros(8), q, k, v, slots, kc, kc.copy(), 4, 2, 64,
                           dtype="f16")
    assert np.array_equal(q_out, q)
    assert np.array_equal(kc2.reshape(-1, 2, 64)[slots], k)
    assert np.array_equal(vc2.reshape(-1, 2, 64)[slots], v)


@pytest.mark.parametrize("is_neox", [True, False])
def test_f16_one_hot_is_rounded_cos_sin(oracle, is_neox):
    """A 1.0 at pair i's first element turns into (cos, sin) of pos * theta^(-2i/D),
    each rounded once to fp16 (numpy's float64 -> float16 rounding)."""
    D, pos = 64, 1234
    for i in (0, 7, 31):
        q = np.zeros((1, 1, D), np.uint16)
        a, b = (i, i + D // 2) if is_neox else (2 * i, 2 * i + 1)
        q[0, 0, a] = 0x3C00
        q_out, _, _ = _run(oracle, [pos], q, q.copy(), q.copy(), [-1], _empty_cache(1, 1, 1, D),
                           _empty_cache(1, 1, 1, D), 1, 1, D, is_neox=is_neox, dtype="f16")
        ang = pos * THETA ** (-2.0 * i / D)
        assert q_out[0, 0, a] == _f16(math.cos(ang)) and q_out[0, 0, b] == _f16(math.sin(ang))
        rest = np.delete(q_out[0, 0], [a, b])
        assert np.all(_f16_to_f64(rest) == 0)  # +0 or -0 (0 * cos - 0 * sin)


@pytest.mark.parametrize("is_neox", [True, False])
def test_f16_agrees_with_bf16_on_shared_values(oracle, is_neox):
    """bf16 inputs in [2^-14, 2^15) are exact fp16 values too.  Both element
    types rotate the same reals in double, so each fp16 output rounded on to
    bf16 is within one bf16 unit of the bf16 output, and v is copied bit for
    bit in either type."""
    T, Hq, Hkv, D, nb, B = 16, 4, 2, 128, 4, 8
    rng = np.random.default_rng(11)

    def shared(shape):
        x = rng.standard_normal(shape)
        x = np.where(np.abs(x) < 2 ** -13, 0.5, x)
        return _bf16(x)

    qb, kb, vb = shared((T, Hq, D)), shared((T, Hkv, D)), shared((T, Hkv, D))
    qh, kh, vh = (_f16(bf16_to_f64(a)) for a in (qb, kb, vb))
    assert np.array_equal(_f16_to_f64(qh), bf16_to_f64(qb))
    pos = rng.integers(0, 4096, T)
    slots = rng.permutation(nb * B)[:T]
    kc = np.zeros((nb, B, Hkv, D), np.uint16)
    ob = _run(oracle, pos, qb, kb, vb, slots, kc, kc.copy(), Hq, Hkv, D, is_neox=is_neox)
    oh = _run(oracle, pos, qh, kh, vh, slots, kc, kc.copy(), Hq, Hkv, D, is_neox=is_neox,
              dtype="f16")
    for got_h, got_b in ((oh[0], ob[0]), (oh[1], ob[1])):
        via = _bf16(_f16_to_f64(got_h)).astype(np.int32)
        sb = got_b.astype(np.int32)
        assert np.max(np.abs(via - sb)) <= 1
        assert np.mean(via == sb) > 0.9
    w = oh[2].reshape(-1, Hkv, D)[slots]
    assert np.array_equal(w, vh)


def test_f16_fused_equals_unfused_and_bad_dtype(oracle):
    rng = np.random.default_rng(3)
    T, Hq, Hkv, D = 8, 2, 1, 64
    q, k, v = _f16(rng.standard_normal((T, Hq, D))), _f16(rng.standard_normal((T, Hkv, D))), \
        _f16(rng.standard_normal((T, Hkv, D)))
    pos, slots = rng.integers(0, 100, T), rng.permutation(16)[:T]
    kc = _empty_cache(2, 8, Hkv, D)
    a = _run(oracle, pos, q, k, v, slots, kc, kc.copy(), Hq, Hkv, D, dtype="f16")
    b = oracle.unfused_rope_kv_write(pos, q, k, v, THETA, 1 << 20, slots, kc, kc.copy(), Hq, Hkv,
                                     D, dtype="f16")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[2])
    assert np.array_equal(a[2], b[3])
    with pytest.raises(ValueError):
        _run(oracle, pos, q, k, v, slots, kc, kc, Hq, Hkv, D, dtype="fp8")
