"""GPU parity: rope_kv_write (and its cos/sin table) against the CPU oracle.

Covers the Llama-3-8B attention workload (32 q / 8 kv heads of 128, theta
500000, positions in [0, 8192), a [4096, 16, 8, 128] bf16 paged cache, slots
drawn without repetition from a seeded permutation; T in {16, 2048, 8192,
16384}), padding tokens (slot -1), in-place and separate q_out, q/k/v as
views of one fused qkv projection, other head sizes and block sizes, ragged
head counts and T = 0, each also with fp16 elements (the same shapes in IEEE
binary16; bar: one fp16 unit) and in the GPT-J pairing.

Bars: rotated q and k within rtol 1e-2 (atol 1e-5) of the oracle; the set of
written cache slots, their placement and the copied v bit-exact; every slot
outside slot_mapping keeps its sentinel bit pattern.  The oracle recomputes
every token at every T; the placement, v copy and sentinel checks run on
every slot."""
import dataclasses

import numpy as np
import pytest

import workloads
from gpu_util import (assert_bf16, assert_elem, dev, dev_bf16, dev_elem, host_bf16, host_f32,
                      require_gpu, compare_rows, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rra():
    require_gpu()
    import rope_residual_add_amd as r

    r.lib()
    return r


def run(rra, oracle, T, cfg=workloads.ROPE, *, pad_every=0, inplace=True, fused_qkv=False):
    import torch

    say(f"[rope] T={T} Hq={cfg.Hq} Hkv={cfg.Hkv} D={cfg.D} blocks={cfg.num_blocks}x"
        f"{cfg.block_size} pad_every={pad_every} inplace={inplace} fused_qkv={fused_qkv} "
        f"neox={cfg.is_neox} dtype={cfg.dtype}")
    dt = cfg.dtype
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    d = workloads.rope_inputs(T, cfg)
    slots = d["slot_mapping"].copy()
    if pad_every:
        slots[::pad_every] = -1
    Hq, Hkv, D = cfg.Hq, cfg.Hkv, cfg.D
    if fused_qkv:
        qkv = np.concatenate([d["q"].reshape(T, -1), d["k"].reshape(T, -1),
                              d["v"].reshape(T, -1)], axis=1)
        qkv_dev = dev_elem(qkv, dt)
        q = qkv_dev[:, :Hq * D]
        k = qkv_dev[:, Hq * D:(Hq + Hkv) * D]
        v = qkv_dev[:, (Hq + Hkv) * D:]
    else:
        q, k, v = dev_elem(d["q"], dt), dev_elem(d["k"], dt), dev_elem(d["v"], dt)
    q_out = None if inplace else torch.empty((T, Hq, D), dtype=tdt, device="cuda")
    kc, vc = dev_elem(d["key_cache"], dt), dev_elem(d["value_cache"], dt)
    cos_sin = rra.rope_cos_sin_cache(cfg.max_pos, cfg.rot_dim, cfg.theta)
    res = rra.rope_kv_write(dev(d["positions"]), q, k, v, cos_sin, dev(slots), kc, vc,
                            q_out=q_out, is_neox=cfg.is_neox)
    torch.cuda.synchronize()
    if inplace:
        assert res.data_ptr() == q.data_ptr()

    n_slots = cfg.num_blocks * cfg.block_size
    gq = host_bf16(res).reshape(T, Hq, D)
    gk = host_bf16(kc).reshape(n_slots, Hkv, D)
    gv = host_bf16(vc).reshape(n_slots, Hkv, D)
    k0 = d["key_cache"].reshape(n_slots, Hkv, D)
    v0 = d["value_cache"].reshape(n_slots, Hkv, D)

    # every slot: untouched outside slot_mapping, v bit-copied inside it
    live = slots >= 0
    written = np.zeros(n_slots, bool)
    written[slots[live]] = True
    assert np.array_equal(gk[~written], k0[~written]), "key cache changed outside slot_mapping"
    assert np.array_equal(gv[~written], v0[~written]), "value cache changed outside slot_mapping"
    assert np.array_equal(gv[slots[live]], d["v"][live]), "value cache != v at the token slots"

    # every token: rotated q and k against the oracle
    rows = compare_rows(T)
    if rows.size == 0:
        return
    ref_q, ref_kc, ref_vc = oracle.rope_kv_write(
        d["positions"][rows], d["q"][rows], d["k"][rows], d["v"][rows], cfg.theta, cfg.max_pos,
        slots[rows], d["key_cache"], d["value_cache"], Hq, Hkv, D, is_neox=cfg.is_neox,
        dtype=dt)
    assert_elem(gq[rows], ref_q, f"q_out T={T}", dt)
    rs = slots[rows]
    rs = rs[rs >= 0]
    ref_kc = ref_kc.reshape(n_slots, Hkv, D)
    ref_vc = ref_vc.reshape(n_slots, Hkv, D)
    assert_elem(gk[rs], ref_kc[rs], f"key cache T={T}", dt)
    assert np.array_equal(gv[rs], ref_vc[rs])


def test_cos_sin_table(rra):
    """cos_sin[p, i] = cos(p * theta^(-2i/128)), cos_sin[p, 64 + i] = sin(same)."""
    say("[rope] cos/sin table")
    c = workloads.ROPE
    tab = host_f32(rra.rope_cos_sin_cache(c.max_pos, c.rot_dim, c.theta))
    p = np.arange(c.max_pos, dtype=np.float64)[:, None]
    i = np.arange(c.rot_dim // 2, dtype=np.float64)[None, :]
    ang = p * c.theta ** (-2.0 * i / c.rot_dim)
    assert np.max(np.abs(tab[:, :64] - np.cos(ang))) < 1e-7
    assert np.max(np.abs(tab[:, 64:] - np.sin(ang))) < 1e-7
    assert np.array_equal(tab[0, :64], np.ones(64, np.float32))
    assert np.array_equal(tab[0, 64:], np.zeros(64, np.float32))


@pytest.mark.parametrize("T", workloads.ROPE.Ts)
def test_attention_workload(rra, oracle, T):
    run(rra, oracle, T)


def test_gptj_at_full_size(rra, oracle):
    """The attention workload at T = 8192 with GPT-J pairs (768 one-vector
    units per token: twelve waves) and padding tokens mixed in."""
    run(rra, oracle, 8192, dataclasses.replace(workloads.ROPE, is_neox=False), pad_every=97)


def test_padding_tokens(rra, oracle):
    run(rra, oracle, 300, pad_every=3)


def test_separate_q_out(rra, oracle):
    run(rra, oracle, 77, inplace=False)


def test_fused_qkv_views(rra, oracle):
    run(rra, oracle, 129, fused_qkv=True)


SMALL = dict(num_blocks=64, max_pos=4096)


@pytest.mark.parametrize("Hq,Hkv,D,bs", [(12, 2, 128, 16), (8, 1, 64, 16), (16, 4, 256, 16),
                                         (40, 8, 128, 1), (33, 3, 64, 32), (64, 8, 128, 16)])
def test_head_and_block_shapes(rra, oracle, Hq, Hkv, D, bs):
    cfg = dataclasses.replace(workloads.ROPE, Hq=Hq, Hkv=Hkv, D=D, rot_dim=D, block_size=bs,
                              **SMALL)
    run(rra, oracle, 45, cfg, pad_every=7)


# GPT-J pairing takes one 16-byte vector (4 pairs) per rotation unit.  A token
# gets one wave per 64 units at one unit per lane, up to 32 waves: these shapes
# give 2, 4, 12, 20 and 28 waves of one unit per lane and, for the last (5120
# units), 27 waves of three units per lane.
@pytest.mark.parametrize("Hq,Hkv,D", [(8, 1, 64), (12, 2, 128), (32, 8, 128), (64, 8, 128),
                                      (40, 8, 256), (128, 16, 256)])
def test_gptj_units_per_pass(rra, oracle, Hq, Hkv, D):
    cfg = dataclasses.replace(workloads.ROPE, Hq=Hq, Hkv=Hkv, D=D, rot_dim=D, is_neox=False,
                              **SMALL)
    run(rra, oracle, 37, cfg, pad_every=5)


@pytest.mark.parametrize("T", [1000, 1365, 171])
def test_partial_xcd_groups(rra, oracle, T):
    """Six waves per token in four-wave workgroups, numbered in groups of 128
    workgroups (16 per XCD): T = 1000 gives 1500 workgroups (92 past the last
    whole group), 1365 gives 2048 (whole groups; the last token ends
    mid-workgroup) and 171 gives 257 (one past)."""
    cfg = dataclasses.replace(workloads.ROPE, num_blocks=128, max_pos=4096)
    run(rra, oracle, T, cfg, pad_every=9)


@pytest.mark.parametrize("neox", [True, False])
def test_multi_pass_tokens(rra, oracle, neox):
    """544 heads of 256: 8704 NeoX or 17408 GPT-J units per token, more than
    32 waves carry at the most units per lane (4 or 8), so each lane loops over
    two passes."""
    cfg = dataclasses.replace(workloads.ROPE, Hq=480, Hkv=32, D=256, rot_dim=256, is_neox=neox,
                              **SMALL)
    run(rra, oracle, 6, cfg, pad_every=4)


@pytest.mark.parametrize("Hq,Hkv,neox", [(65536, 1, True), (65536, 1, False), (1, 65536, True)])
def test_largest_head_counts(rra, oracle, Hq, Hkv, neox):
    """The largest head counts the entry point takes, which the kernel receives
    packed as (Hq - 1) | (Hkv - 1) << 16: 65536 heads of 64 fill both 16-bit
    fields and give each lane many passes at the most units per pass."""
    cfg = dataclasses.replace(workloads.ROPE, Hq=Hq, Hkv=Hkv, D=64, rot_dim=64, is_neox=neox,
                              num_blocks=1, block_size=4, max_pos=4096)
    run(rra, oracle, 3, cfg, pad_every=3)


def test_position_zero_is_identity(rra):
    """At position 0 the rotation is the identity: q_out == q, cache == k."""
    import torch

    say("[rope] position 0")
    c = dataclasses.replace(workloads.ROPE, **SMALL)
    d = workloads.rope_inputs(20, c)
    pos = np.zeros(20, np.int64)
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    kc, vc = dev_bf16(d["key_cache"]), dev_bf16(d["value_cache"])
    cs = rra.rope_cos_sin_cache(c.max_pos, c.rot_dim, c.theta)
    rra.rope_kv_write(dev(pos), q, k, v, cs, dev(d["slot_mapping"]), kc, vc)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(q), d["q"])
    n = c.num_blocks * c.block_size
    assert np.array_equal(host_bf16(kc).reshape(n, c.Hkv, c.D)[d["slot_mapping"]], d["k"])


def test_empty(rra):
    import torch

    say("[rope] T=0")
    c = dataclasses.replace(workloads.ROPE, **SMALL)
    e = lambda *s: torch.empty(s, dtype=torch.bfloat16, device="cuda")
    i = torch.empty(0, dtype=torch.int64, device="cuda")
    kc = e(c.num_blocks, c.block_size, c.Hkv, c.D)
    cs = rra.rope_cos_sin_cache(c.max_pos, c.rot_dim, c.theta)
    out = rra.rope_kv_write(i, e(0, c.Hq, c.D), e(0, c.Hkv, c.D), e(0, c.Hkv, c.D), cs, i, kc,
                            kc.clone())
    assert out.shape == (0, c.Hq, c.D)


F16 = dataclasses.replace(workloads.ROPE, dtype="f16")


@pytest.mark.parametrize("T", workloads.ROPE_F16.Ts)
def test_f16_attention_workload(rra, oracle, T):
    run(rra, oracle, T, workloads.ROPE_F16)


@pytest.mark.parametrize("is_neox", [True, False])
def test_f16_padding_separate_out_and_gptj(rra, oracle, is_neox):
    run(rra, oracle, 200, dataclasses.replace(F16, is_neox=is_neox), pad_every=4, inplace=False)


def test_f16_fused_qkv_views(rra, oracle):
    run(rra, oracle, 65, F16, fused_qkv=True)


@pytest.mark.parametrize("Hq,Hkv,D,bs", [(8, 1, 64, 16), (16, 4, 256, 8), (33, 3, 64, 32)])
def test_f16_head_and_block_shapes(rra, oracle, Hq, Hkv, D, bs):
    cfg = dataclasses.replace(F16, Hq=Hq, Hkv=Hkv, D=D, rot_dim=D, block_size=bs, **SMALL)
    run(rra, oracle, 45, cfg, pad_every=7)


def test_f16_empty_and_mixed_types_rejected(rra):
    import torch

    say("[rope] fp16 T=0 and mixed element types")
    c = dataclasses.replace(F16, **SMALL)
    e = lambda *s, dt=torch.float16: torch.empty(s, dtype=dt, device="cuda")
    i = torch.empty(0, dtype=torch.int64, device="cuda")
    kc = e(c.num_blocks, c.block_size, c.Hkv, c.D)
    cs = rra.rope_cos_sin_cache(c.max_pos, c.rot_dim, c.theta)
    out = rra.rope_kv_write(i, e(0, c.Hq, c.D), e(0, c.Hkv, c.D), e(0, c.Hkv, c.D), cs, i, kc,
                            kc.clone())
    assert out.shape == (0, c.Hq, c.D) and out.dtype == torch.float16
    with pytest.raises(TypeError):  # bf16 k with fp16 q: refused on the host
        rra.rope_kv_write(i, e(0, c.Hq, c.D), e(0, c.Hkv, c.D, dt=torch.bfloat16),
                          e(0, c.Hkv, c.D), cs, i, kc, kc.clone())
