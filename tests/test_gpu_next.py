"""GPU parity for the next rows against the CPU oracle:

- qk_norm_rope_kv_write: Qwen3-style attention (32 q / 8 kv heads of 128,
  theta 1e6, eps 1e-6) on the packed qkv rows, with the paged cache write
  (T in {16, 2048, 8192}), without a cache and with k written back, GPT-J
  pairing, other head sizes, padding tokens, T = 0.
- fused_add_rmsnorm_pad: GPT-OSS hidden 2880 padded to 3072 (T in {16, 2048,
  8192}), without residual, other widths, T = 0.
- mla_rope_kv_write: DeepSeek-V3 MLA (128 heads of nope 128 + rope 64, kv_lora
  512, GPT-J pairing, 576-wide cache rows; T in {16, 2048, 8192}), neox
  pairing, padding tokens, T = 0.

Bars as for the other kernels: bf16 outputs within rtol 1e-2 (atol 1e-5);
cache placement, copied values, untouched columns and untouched slots
bit-exact.  Every token is compared with the oracle at every T, and the
placement and untouched-slot properties are checked on every slot."""
import dataclasses

import numpy as np
import pytest

import workloads
from gpu_util import (assert_bf16, assert_elem, dev, dev_bf16, dev_elem, host_bf16, require_gpu,
                      compare_rows, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rra():
    require_gpu()
    import rope_residual_add_amd as r

    r.lib()
    return r


# ---- QK norm + RoPE (+ KV write) ----------------------------------------------------

def run_qknorm(rra, oracle, T, cfg=workloads.QKNORM, *, cache=True, write_k=False, is_neox=True,
               pad_every=0):
    import torch

    say(f"[qknorm] T={T} Hq={cfg.Hq} Hkv={cfg.Hkv} D={cfg.D} cache={cache} write_k={write_k} "
        f"neox={is_neox} pad_every={pad_every}")
    d = workloads.qknorm_inputs(T, cfg, with_cache=cache)
    slots = d["slot_mapping"].copy()
    if pad_every:
        slots[::pad_every] = -1
    Hq, Hkv, D = cfg.Hq, cfg.Hkv, cfg.D
    qkv = dev_bf16(d["qkv"])
    cs = rra.rope_cos_sin_cache(cfg.max_pos, D, cfg.theta)
    kc = dev_bf16(d["key_cache"]) if cache else None
    vc = dev_bf16(d["value_cache"]) if cache else None
    rra.qk_norm_rope_kv_write(dev(d["positions"]), qkv, dev_bf16(d["q_w"]), dev_bf16(d["k_w"]),
                              cfg.eps, cs, Hq, Hkv, D, slot_mapping=dev(slots) if cache else None,
                              key_cache=kc, value_cache=vc, write_k=write_k, is_neox=is_neox)
    torch.cuda.synchronize()
    g = host_bf16(qkv)
    qc, kcols = Hq * D, (Hq + Hkv) * D
    # every token: v untouched; k untouched unless written back
    assert np.array_equal(g[:, kcols:], d["qkv"][:, kcols:]), "v part of qkv changed"
    if not write_k:
        assert np.array_equal(g[:, qc:kcols], d["qkv"][:, qc:kcols]), "k part of qkv changed"
    if cache:
        n = cfg.num_blocks * cfg.block_size
        gk, gv = host_bf16(kc).reshape(n, Hkv, D), host_bf16(vc).reshape(n, Hkv, D)
        k0, v0 = d["key_cache"].reshape(n, Hkv, D), d["value_cache"].reshape(n, Hkv, D)
        live = slots >= 0
        written = np.zeros(n, bool)
        written[slots[live]] = True
        assert np.array_equal(gk[~written], k0[~written]), "key cache changed outside slots"
        assert np.array_equal(gv[~written], v0[~written]), "value cache changed outside slots"
        v_in = d["qkv"][:, kcols:].reshape(T, Hkv, D)
        assert np.array_equal(gv[slots[live]], v_in[live]), "value cache != v"
    rows = compare_rows(T)
    if rows.size == 0:
        return
    kw = dict(write_k=write_k, is_neox=is_neox)
    if cache:
        kw.update(slot_mapping=slots[rows], key_cache=d["key_cache"],
                  value_cache=d["value_cache"])
    ref, ref_kc, _ = oracle.qk_norm_rope_kv_write(d["positions"][rows], d["qkv"][rows],
                                                  d["q_w"], d["k_w"], cfg.eps, cfg.theta,
                                                  cfg.max_pos, Hq, Hkv, D, **kw)
    assert_bf16(g[rows, :qc], ref[:, :qc], f"q T={T}")
    if write_k:
        assert_bf16(g[rows, qc:kcols], ref[:, qc:kcols], f"k written back T={T}")
    if cache:
        rs = slots[rows]
        rs = rs[rs >= 0]
        n = cfg.num_blocks * cfg.block_size
        assert_bf16(gk[rs], ref_kc.reshape(n, Hkv, D)[rs], f"key cache T={T}")


@pytest.mark.parametrize("T", workloads.QKNORM.Ts)
def test_qknorm_workload(rra, oracle, T):
    run_qknorm(rra, oracle, T)


QK_SMALL = dict(num_blocks=64, max_pos=4096)


def test_qknorm_no_cache_write_k(rra, oracle):
    run_qknorm(rra, oracle, 37, cache=False, write_k=True)


def test_qknorm_cache_and_write_k_padding(rra, oracle):
    cfg = dataclasses.replace(workloads.QKNORM, **QK_SMALL)
    run_qknorm(rra, oracle, 100, cfg, write_k=True, pad_every=4)


@pytest.mark.parametrize("Hq,Hkv,D,neox", [(32, 8, 128, False), (16, 4, 64, True),
                                           (8, 2, 256, True), (12, 3, 64, False),
                                           (8, 2, 256, False), (64, 8, 128, False),
                                           (96, 16, 128, False)])
def test_qknorm_shapes(rra, oracle, Hq, Hkv, D, neox):
    cfg = dataclasses.replace(workloads.QKNORM, Hq=Hq, Hkv=Hkv, D=D, **QK_SMALL)
    run_qknorm(rra, oracle, 41, cfg, is_neox=neox, pad_every=5)


@pytest.mark.parametrize("neox", [True, False])
def test_qknorm_multi_pass_tokens(rra, oracle, neox):
    """480 q and 32 kv heads of 256 with a cache: 8704 NeoX or 17408 GPT-J
    units per token, two passes per lane at the most units per lane."""
    cfg = dataclasses.replace(workloads.QKNORM, Hq=480, Hkv=32, D=256, **QK_SMALL)
    run_qknorm(rra, oracle, 5, cfg, is_neox=neox, write_k=True, pad_every=3)


@pytest.mark.parametrize("Hq,Hkv", [(65536, 1), (1, 65536)])
def test_qknorm_largest_head_counts(rra, oracle, Hq, Hkv):
    """Head counts of 65536, the most the entry point takes (packed for the
    kernel as (Hq - 1) | (Hkv - 1) << 16), with a cache and k written back."""
    cfg = dataclasses.replace(workloads.QKNORM, Hq=Hq, Hkv=Hkv, D=64, num_blocks=1, block_size=4,
                              max_pos=4096)
    run_qknorm(rra, oracle, 3, cfg, cache=True, write_k=True, pad_every=3)


def test_qknorm_empty(rra):
    import torch

    say("[qknorm] T=0")
    c = workloads.QKNORM
    qkv = torch.empty((0, (c.Hq + 2 * c.Hkv) * c.D), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(c.D, dtype=torch.bfloat16, device="cuda")
    cs = rra.rope_cos_sin_cache(16, c.D, c.theta)
    pos = torch.empty(0, dtype=torch.int64, device="cuda")
    out = rra.qk_norm_rope_kv_write(pos, qkv, w, w, c.eps, cs, c.Hq, c.Hkv, c.D)
    assert out.shape == qkv.shape


# ---- residual add + RMSNorm + padding ---------------------------------------------

def run_pad(rra, oracle, T, H, H_pad, residual=True, eps=1e-5, dtype="bf16"):
    import torch

    say(f"[pad] T={T} H={H} H_pad={H_pad} residual={residual} dtype={dtype}")
    d = workloads.norm_inputs(T, H, tag="pad", dtype=dtype)
    x = dev_elem(d["x"], dtype)
    r = dev_elem(d["residual"], dtype) if residual else None
    r0 = r.clone() if residual else None
    out = rra.fused_add_rmsnorm_pad(x, r, dev_elem(d["weight"], dtype), eps, H_pad)
    torch.cuda.synchronize()
    assert out.dtype == x.dtype
    g = host_bf16(out)
    assert np.array_equal(g[:, H:], np.zeros((T, H_pad - H), np.uint16)), "pad columns not +0"
    if residual:
        # fp32 carries 2p + 2 bits for both types, so this is the exact sum rounded once
        full = (x.float() + r0.float()).to(x.dtype)
        assert torch.equal(full.view(torch.int16), r.view(torch.int16))
    rows = compare_rows(T)
    if rows.size == 0:
        return
    ref, ref_res = oracle.fused_add_rmsnorm_pad(d["x"][rows],
                                                d["residual"][rows] if residual else None,
                                                d["weight"], eps, H_pad, dtype=dtype)
    assert_elem(g[rows], ref, f"normed T={T} H={H}", dtype)
    if residual:
        assert np.array_equal(host_bf16(r)[rows], ref_res)


@pytest.mark.parametrize("T", workloads.PAD.Ts)
def test_pad_workload(rra, oracle, T):
    run_pad(rra, oracle, T, workloads.PAD.H, workloads.PAD.H_pad, eps=workloads.PAD.eps)


@pytest.mark.parametrize("T,H,H_pad,residual", [(9, 2880, 3072, False), (33, 1000, 1024, True),
                                                (7, 4096, 4096, True), (5, 8, 64, True),
                                                (3, 2048, 2304, True)])
def test_pad_shapes(rra, oracle, T, H, H_pad, residual):
    run_pad(rra, oracle, T, H, H_pad, residual)


@pytest.mark.parametrize("T", workloads.PAD_F16.Ts)
def test_pad_f16_workload(rra, oracle, T):
    c = workloads.PAD_F16
    run_pad(rra, oracle, T, c.H, c.H_pad, eps=c.eps, dtype="f16")


@pytest.mark.parametrize("T,H,H_pad,residual", [(9, 2880, 3072, False), (33, 1000, 1024, True),
                                                (5, 8, 64, True), (3, 8192, 8192, True)])
def test_pad_f16_shapes(rra, oracle, T, H, H_pad, residual):
    run_pad(rra, oracle, T, H, H_pad, residual, dtype="f16")


def test_pad_empty(rra):
    import torch

    say("[pad] T=0")
    x = torch.empty((0, 2880), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(2880, dtype=torch.bfloat16, device="cuda")
    out = rra.fused_add_rmsnorm_pad(x, None, w, 1e-5, 3072)
    assert out.shape == (0, 3072)


# ---- MLA RoPE + [kv_c | k_pe] cache write -------------------------------------------

def run_mla_rope(rra, oracle, T, cfg=workloads.MLA_ROPE, pad_every=0):
    import torch

    say(f"[mla_rope] T={T} Hq={cfg.Hq} rope={cfg.rope_dim} neox={cfg.is_neox} "
        f"pad_every={pad_every}")
    d = workloads.mla_rope_inputs(T, cfg)
    slots = d["slot_mapping"].copy()
    if pad_every:
        slots[::pad_every] = -1
    hs = cfg.nope + cfg.rope_dim
    q = dev_bf16(d["q"])
    cache = dev_bf16(d["kv_cache"])
    cs = rra.rope_cos_sin_cache(cfg.max_pos, cfg.rope_dim, cfg.theta)
    rra.mla_rope_kv_write(dev(d["positions"]), q, dev_bf16(d["k_pe"]), dev_bf16(d["kv_c"]), cs,
                          dev(slots), cache, cfg.Hq, cfg.rope_dim, hs, cfg.nope,
                          is_neox=cfg.is_neox)
    torch.cuda.synchronize()
    gq = host_bf16(q).reshape(T, cfg.Hq, hs)
    assert np.array_equal(gq[:, :, :cfg.nope], d["q"].reshape(T, cfg.Hq, hs)[:, :, :cfg.nope]), \
        "nope part of q changed"
    n = cfg.num_blocks * cfg.block_size
    w = cfg.kv_lora + cfg.rope_dim
    gc, c0 = host_bf16(cache).reshape(n, w), d["kv_cache"].reshape(n, w)
    live = slots >= 0
    written = np.zeros(n, bool)
    written[slots[live]] = True
    assert np.array_equal(gc[~written], c0[~written]), "cache changed outside slots"
    assert np.array_equal(gc[slots[live], :cfg.kv_lora], d["kv_c"][live]), "kv_c not copied"
    rows = compare_rows(T)
    if rows.size == 0:
        return
    ref_q, ref_c = oracle.mla_rope_kv_write(d["positions"][rows], d["q"][rows], d["k_pe"][rows],
                                            d["kv_c"][rows], cfg.theta, cfg.max_pos, slots[rows],
                                            d["kv_cache"], cfg.Hq, cfg.rope_dim, q_head_stride=hs,
                                            q_pe_offset=cfg.nope, is_neox=cfg.is_neox)
    assert_bf16(gq[rows][:, :, cfg.nope:], ref_q.reshape(-1, cfg.Hq, hs)[:, :, cfg.nope:],
                f"q_pe T={T}")
    rs = slots[rows]
    rs = rs[rs >= 0]
    assert_bf16(gc[rs, cfg.kv_lora:], ref_c.reshape(n, w)[rs, cfg.kv_lora:], f"k_pe T={T}")


@pytest.mark.parametrize("T", workloads.MLA_ROPE.Ts)
def test_mla_rope_workload(rra, oracle, T):
    run_mla_rope(rra, oracle, T)


@pytest.mark.parametrize("Hq,rope,neox", [(16, 64, True), (7, 128, False), (1, 64, False),
                                           (256, 64, False), (128, 128, False)])
def test_mla_rope_shapes(rra, oracle, Hq, rope, neox):
    cfg = dataclasses.replace(workloads.MLA_ROPE, Hq=Hq, rope_dim=rope, is_neox=neox,
                              num_blocks=16, max_pos=2048)
    run_mla_rope(rra, oracle, 57, cfg, pad_every=6)


@pytest.mark.parametrize("neox", [True, False])
def test_mla_rope_multi_pass_tokens(rra, oracle, neox):
    """2100 heads: 8468 NeoX or 16872 GPT-J units per token (with kv_c's 64
    copy units), two passes per lane at the most units per lane."""
    cfg = dataclasses.replace(workloads.MLA_ROPE, Hq=2100, is_neox=neox, num_blocks=16,
                              max_pos=2048)
    run_mla_rope(rra, oracle, 5, cfg, pad_every=3)


def test_mla_rope_empty(rra):
    import torch

    say("[mla_rope] T=0")
    c = workloads.MLA_ROPE
    e = lambda *s: torch.empty(s, dtype=torch.bfloat16, device="cuda")
    i = torch.empty(0, dtype=torch.int64, device="cuda")
    cache = e(2, c.block_size, c.kv_lora + c.rope_dim)
    cs = rra.rope_cos_sin_cache(16, c.rope_dim, c.theta)
    q = rra.mla_rope_kv_write(i, e(0, c.Hq * (c.nope + c.rope_dim)), e(0, c.rope_dim),
                              e(0, c.kv_lora), cs, i, cache, c.Hq, c.rope_dim,
                              c.nope + c.rope_dim, c.nope)
    assert q.shape[0] == 0
