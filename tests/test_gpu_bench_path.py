"""Parity of the exact launch path bench.py times: its launchers, buffers and
device-generated inputs at the full workload sizes (T = 8192), one launch of
every kernel, every token checked against the CPU oracle with the same bars
as the other GPU tests.  For the cache-writing kernels the tokens' slots are
remapped onto a compact oracle cache, one slot per token (a written slot
depends only on its own token)."""
import numpy as np
import pytest

import workloads
from gpu_util import assert_bf16, assert_codes, assert_elem, assert_scales, require_gpu, say

pytestmark = pytest.mark.gpu

T = 8192


@pytest.fixture(scope="module")
def launchers():
    require_gpu()
    import bench

    return bench.make_launchers(T, salt=7, only=bench.KERNELS + bench.NEXT_KERNELS)


@pytest.fixture(scope="module")
def rows():
    return np.arange(T)


def h16(t, rows=None):
    import torch

    if rows is not None:
        t = t[torch.as_tensor(rows, device=t.device)]
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def h8(t, rows):
    import torch

    return t[torch.as_tensor(rows, device=t.device)].contiguous().view(torch.uint8).cpu().numpy()


def hf(t, rows):
    import torch

    return t[torch.as_tensor(rows, device=t.device)].cpu().numpy()


def hi(t, rows=None):
    import torch

    if rows is not None:
        t = t[torch.as_tensor(rows, device=t.device)]
    return t.cpu().numpy()


def launch(launchers, name):
    import torch

    say(f"[bench path] {name} T={T}")
    launchers[name]()
    torch.cuda.synchronize()


def test_norm(launchers, rows, oracle):
    io = launchers["_io"]["fused_add_rmsnorm_quant"]
    x, r, w = h16(io["x"], rows), h16(io["residual"], rows), h16(io["weight"])
    launch(launchers, "fused_add_rmsnorm_quant")
    codes, scales, res = oracle.fused_add_rmsnorm_quant(x, r, w, 1e-5, oracle.Q_PER_TOKEN)
    assert_codes(h8(io["out"], rows), codes, "bench-path norm codes", exact=True)
    assert_scales(hf(io["scales"], rows), scales, "bench-path norm scales")
    assert np.array_equal(h16(io["residual"], rows), res)


def test_silu(launchers, rows, oracle):
    io = launchers["_io"]["silu_mul_quant"]
    inp = h16(io["inp"], rows)
    launch(launchers, "silu_mul_quant")
    codes, scales = oracle.silu_mul_quant(inp, oracle.Q_PER_GROUP, 128)
    assert_codes(h8(io["out"], rows), codes, "bench-path silu codes")
    assert_scales(hf(io["scales"], rows), scales, "bench-path silu scales")


def test_mla(launchers, rows, oracle):
    io = launchers["_io"]["dual_rmsnorm_quant"]
    q, kv = h16(io["q"], rows), h16(io["kv"], rows)
    qw, kvw = h16(io["q_w"]), h16(io["kv_w"])
    launch(launchers, "dual_rmsnorm_quant")
    rq, rs, rkv = oracle.dual_rmsnorm_quant(q, qw, 1e-6, kv, kvw, 1e-6, oracle.Q_PER_GROUP, 128)
    assert_codes(h8(io["q_out"], rows), rq, "bench-path mla q codes", exact=True)
    assert_scales(hf(io["q_scales"], rows), rs, "bench-path mla q scales")
    assert_bf16(h16(io["kv_out"], rows), rkv, "bench-path mla kv")


def _compact_cache(shape_tail, n):
    return np.zeros((n, 1) + tuple(shape_tail), np.uint16)


@pytest.mark.parametrize("name,c", [("rope_kv_write", workloads.ROPE),
                                    ("rope_kv_write_f16", workloads.ROPE_F16)])
def test_rope(launchers, rows, oracle, name, c):
    io = launchers["_io"][name]
    q, k, v = h16(io["q"], rows), h16(io["k"], rows), h16(io["v"], rows)
    pos, slots = hi(io["positions"], rows), hi(io["slot_mapping"], rows)
    launch(launchers, name)
    n = len(rows)
    kc0 = _compact_cache((c.Hkv, c.D), n)
    ref_q, ref_kc, ref_vc = oracle.rope_kv_write(pos, q, k, v, c.theta, c.max_pos, np.arange(n),
                                                 kc0, kc0, c.Hq, c.Hkv, c.D, dtype=c.dtype)
    assert_elem(h16(io["q"], rows), ref_q, f"bench-path {name} q", c.dtype)
    nb = c.num_blocks * c.block_size
    gk = h16(io["key_cache"]).reshape(nb, c.Hkv, c.D)[slots]
    gv = h16(io["value_cache"]).reshape(nb, c.Hkv, c.D)[slots]
    assert_elem(gk, ref_kc.reshape(n, c.Hkv, c.D), f"bench-path {name} key cache", c.dtype)
    assert np.array_equal(gv, ref_vc.reshape(n, c.Hkv, c.D))


def test_qknorm(launchers, rows, oracle):
    c = workloads.QKNORM
    io = launchers["_io"]["qk_norm_rope_kv_write"]
    qkv = h16(io["qkv"], rows)
    qw, kw = h16(io["q_w"]), h16(io["k_w"])
    pos, slots = hi(io["positions"], rows), hi(io["slot_mapping"], rows)
    launch(launchers, "qk_norm_rope_kv_write")
    n = len(rows)
    kc0 = _compact_cache((c.Hkv, c.D), n)
    ref, ref_kc, ref_vc = oracle.qk_norm_rope_kv_write(pos, qkv, qw, kw, c.eps, c.theta,
                                                       c.max_pos, c.Hq, c.Hkv, c.D,
                                                       slot_mapping=np.arange(n), key_cache=kc0,
                                                       value_cache=kc0)
    g = h16(io["qkv"], rows)
    qc = c.Hq * c.D
    assert_bf16(g[:, :qc], ref[:, :qc], "bench-path qknorm q")
    assert np.array_equal(g[:, qc:], qkv[:, qc:])
    nb = c.num_blocks * c.block_size
    gk = h16(io["key_cache"]).reshape(nb, c.Hkv, c.D)[slots]
    gv = h16(io["value_cache"]).reshape(nb, c.Hkv, c.D)[slots]
    assert_bf16(gk, ref_kc.reshape(n, c.Hkv, c.D), "bench-path qknorm key cache")
    assert np.array_equal(gv, ref_vc.reshape(n, c.Hkv, c.D))


@pytest.mark.parametrize("name,c", [("fused_add_rmsnorm_pad", workloads.PAD),
                                    ("fused_add_rmsnorm_pad_f16", workloads.PAD_F16)])
def test_pad(launchers, rows, oracle, name, c):
    io = launchers["_io"][name]
    x, r, w = h16(io["x"], rows), h16(io["residual"], rows), h16(io["weight"])
    launch(launchers, name)
    ref, ref_res = oracle.fused_add_rmsnorm_pad(x, r, w, c.eps, c.H_pad, dtype=c.dtype)
    assert_elem(h16(io["out"], rows), ref, f"bench-path {name}", c.dtype)
    assert np.array_equal(h16(io["residual"], rows), ref_res)


def test_mla_rope(launchers, rows, oracle):
    c = workloads.MLA_ROPE
    io = launchers["_io"]["mla_rope_kv_write"]
    q, k_pe, kv_c = h16(io["q"], rows), h16(io["k_pe"], rows), h16(io["kv_c"], rows)
    pos, slots = hi(io["positions"], rows), hi(io["slot_mapping"], rows)
    launch(launchers, "mla_rope_kv_write")
    n = len(rows)
    w = c.kv_lora + c.rope_dim
    cache0 = np.zeros((n, 1, w), np.uint16)
    ref_q, ref_c = oracle.mla_rope_kv_write(pos, q, k_pe, kv_c, c.theta, c.max_pos,
                                            np.arange(n), cache0, c.Hq, c.rope_dim,
                                            q_head_stride=c.nope + c.rope_dim,
                                            q_pe_offset=c.nope, is_neox=c.is_neox)
    assert_bf16(h16(io["q"], rows), ref_q, "bench-path mla_rope q")
    nb = c.num_blocks * c.block_size
    g = h16(io["kv_cache"]).reshape(nb, w)[slots]
    assert np.array_equal(g[:, :c.kv_lora], ref_c.reshape(n, w)[:, :c.kv_lora])
    assert_bf16(g[:, c.kv_lora:], ref_c.reshape(n, w)[:, c.kv_lora:], "bench-path mla_rope k_pe")
