"""The C ABI from plain C: tests/c_client/rra_c_client.c includes only
include/rra.h and the HIP runtime API, links librra.so and calls all seven
entry points (plus rope_cos_sin_cache and six calls that must fail on the host
with their documented statuses).  Here it runs as a child process on inputs
written to files, and every output it writes back must be byte-identical to
the Python binding's on the same inputs: one library, two callers.  The
binding's own parity with the oracle is covered by the per-kernel GPU tests.

Without a GPU, the client is checked to build, resolve librra.so through its
run path, match the header's ABI version and reject a bad command line."""
import dataclasses
import os
import subprocess

import numpy as np
import pytest

import workloads
from gpu_util import dev, dev_bf16, host_bf16, host_f32, host_u8, require_gpu, say

HERE = os.path.dirname(os.path.abspath(__file__))
CLIENT_DIR = os.path.join(HERE, "c_client")

# Small cases of the step workloads: a ragged token count for the norm, the
# full Llama-3-8B SiLU width, the headline RoPE heads over a 64-block cache,
# and the DeepSeek-V3 MLA latents.
T_NORM, H_NORM = 33, 4096
T_SILU, I_SILU = 9, 14336
ROPE = workloads.RopeCfg("rope_c_client", num_blocks=64)
T_ROPE = 17
T_MLA = 5
# The next rows at their workload shapes, over smaller caches.
QK = dataclasses.replace(workloads.QKNORM, num_blocks=64)
T_QK = 13
PAD = workloads.PAD
T_PAD = 11
MR = dataclasses.replace(workloads.MLA_ROPE, num_blocks=16)
T_MR = 7


def client_binary() -> str:
    import importlib.util

    spec = importlib.util.spec_from_file_location("rra_c_client_build",
                                                  os.path.join(CLIENT_DIR, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    if not os.path.exists(mod.BINARY):
        import rope_residual_add_amd as r

        if not os.path.exists(r.LIBRARY_PATH):
            from rope_residual_add_amd import build

            build.build()
        mod.build()
    return mod.BINARY


def test_client_links_and_checks_its_command_line(tmp_path):
    exe = client_binary()
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "usage" in r.stderr, (r.returncode, r.stderr)
    # The ABI version is checked before the shapes file is opened.
    r = subprocess.run([exe, str(tmp_path / "missing")], capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 1 and "shapes.txt: cannot open" in r.stderr, (r.returncode, r.stderr)


@pytest.mark.gpu
def test_c_client_matches_the_binding(tmp_path):
    require_gpu()
    import torch

    import rope_residual_add_amd as rra

    exe = client_binary()
    rra.lib()
    nd = workloads.norm_inputs(T_NORM, H_NORM, salt=11)
    sd = workloads.silu_inputs(T_SILU, I_SILU, salt=11)
    rd = workloads.rope_inputs(T_ROPE, ROPE, salt=11)
    md = workloads.mla_inputs(T_MLA, salt=11)
    qd = workloads.qknorm_inputs(T_QK, QK, salt=11)
    pd = workloads.pad_inputs(T_PAD, PAD, salt=11)
    rm = workloads.mla_rope_inputs(T_MR, MR, salt=11)
    files = dict(norm_x=nd["x"], norm_res=nd["residual"], norm_w=nd["weight"],
                 silu_in=sd["inp"], rope_q=rd["q"], rope_k=rd["k"], rope_v=rd["v"],
                 rope_pos=rd["positions"], rope_slot=rd["slot_mapping"],
                 rope_kc=rd["key_cache"], rope_vc=rd["value_cache"], mla_q=md["q"],
                 mla_kv=md["kv"], mla_qw=md["q_w"], mla_kvw=md["kv_w"], qk_qkv=qd["qkv"],
                 qk_qw=qd["q_w"], qk_kw=qd["k_w"], qk_pos=qd["positions"],
                 qk_slot=qd["slot_mapping"], qk_kc=qd["key_cache"], qk_vc=qd["value_cache"],
                 pad_x=pd["x"], pad_res=pd["residual"], pad_w=pd["weight"], mr_q=rm["q"],
                 mr_kpe=rm["k_pe"], mr_kvc=rm["kv_c"], mr_pos=rm["positions"],
                 mr_slot=rm["slot_mapping"], mr_cache=rm["kv_cache"])
    for name, a in files.items():
        np.ascontiguousarray(a).tofile(tmp_path / f"{name}.bin")
    cfg = workloads.MLA
    shapes = [T_NORM, H_NORM, T_SILU, I_SILU, T_ROPE, ROPE.Hq, ROPE.Hkv, ROPE.D,
              ROPE.num_blocks, ROPE.block_size, ROPE.max_pos, int(ROPE.theta), T_MLA, cfg.Hq,
              cfg.Hkv, T_QK, QK.Hq, QK.Hkv, QK.D, QK.num_blocks, QK.block_size, QK.max_pos,
              int(QK.theta), T_PAD, PAD.H, PAD.H_pad, T_MR, MR.Hq, MR.nope, MR.rope_dim,
              MR.kv_lora, MR.num_blocks, MR.block_size, MR.max_pos, int(MR.theta),
              int(MR.is_neox)]
    (tmp_path / "shapes.txt").write_text(" ".join(str(s) for s in shapes) + "\n")

    say(f"[c_client] {exe} on {tmp_path}")
    r = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, timeout=120)
    print(r.stdout + r.stderr, flush=True)
    assert r.returncode == 0, r.stderr

    def out(name, dtype):
        return np.fromfile(tmp_path / f"out_{name}.bin", dtype=dtype)

    say("[c_client] the same calls through the Python binding")
    res = dev_bf16(nd["residual"])
    codes, scales = rra.fused_add_rmsnorm_quant(dev_bf16(nd["x"]), res, dev_bf16(nd["weight"]),
                                                1e-5, "per_token")
    scodes, sscales = rra.silu_mul_quant(dev_bf16(sd["inp"]), "per_group", 128)
    cos_sin = rra.rope_cos_sin_cache(ROPE.max_pos, ROPE.D, ROPE.theta)
    q = dev_bf16(rd["q"])
    kc, vc = dev_bf16(rd["key_cache"]), dev_bf16(rd["value_cache"])
    rra.rope_kv_write(dev(rd["positions"]), q, dev_bf16(rd["k"]), dev_bf16(rd["v"]), cos_sin,
                      dev(rd["slot_mapping"]), kc, vc)
    mq, mqs, mkv = rra.dual_rmsnorm_quant(dev_bf16(md["q"]), dev_bf16(md["q_w"]), cfg.eps_q,
                                          dev_bf16(md["kv"]), dev_bf16(md["kv_w"]), cfg.eps_kv,
                                          "per_group", 128)
    qkv = dev_bf16(qd["qkv"])
    qkc, qvc = dev_bf16(qd["key_cache"]), dev_bf16(qd["value_cache"])
    rra.qk_norm_rope_kv_write(dev(qd["positions"]), qkv, dev_bf16(qd["q_w"]),
                              dev_bf16(qd["k_w"]), QK.eps,
                              rra.rope_cos_sin_cache(QK.max_pos, QK.D, QK.theta), QK.Hq, QK.Hkv,
                              QK.D, slot_mapping=dev(qd["slot_mapping"]), key_cache=qkc,
                              value_cache=qvc, write_k=True)
    pres = dev_bf16(pd["residual"])
    pout = rra.fused_add_rmsnorm_pad(dev_bf16(pd["x"]), pres, dev_bf16(pd["weight"]), PAD.eps,
                                     PAD.H_pad)
    mrq, mrc = dev_bf16(rm["q"]), dev_bf16(rm["kv_cache"])
    rra.mla_rope_kv_write(dev(rm["positions"]), mrq, dev_bf16(rm["k_pe"]), dev_bf16(rm["kv_c"]),
                          rra.rope_cos_sin_cache(MR.max_pos, MR.rope_dim, MR.theta),
                          dev(rm["slot_mapping"]), mrc, MR.Hq, MR.rope_dim,
                          q_head_stride=MR.nope + MR.rope_dim, q_pe_offset=MR.nope,
                          is_neox=MR.is_neox)
    torch.cuda.synchronize()

    pairs = [
        ("norm codes", out("norm_codes", np.uint8), host_u8(codes).ravel()),
        ("norm scales", out("norm_scales", np.float32), host_f32(scales).ravel()),
        ("norm residual", out("norm_res", np.uint16), host_bf16(res).ravel()),
        ("silu codes", out("silu_codes", np.uint8), host_u8(scodes).ravel()),
        ("silu scales", out("silu_scales", np.float32), host_f32(sscales).ravel()),
        ("rope cos/sin table", out("rope_cos_sin", np.float32), host_f32(cos_sin).ravel()),
        ("rope q (in place)", out("rope_q", np.uint16), host_bf16(q).ravel()),
        ("rope key cache", out("rope_kc", np.uint16), host_bf16(kc).ravel()),
        ("rope value cache", out("rope_vc", np.uint16), host_bf16(vc).ravel()),
        ("mla q codes", out("mla_q", np.uint8), host_u8(mq).ravel()),
        ("mla q scales", out("mla_qs", np.float32), host_f32(mqs).ravel()),
        ("mla kv", out("mla_kv", np.uint16), host_bf16(mkv).ravel()),
        ("qk norm qkv (q and k in place)", out("qk_qkv", np.uint16), host_bf16(qkv).ravel()),
        ("qk norm key cache", out("qk_kc", np.uint16), host_bf16(qkc).ravel()),
        ("qk norm value cache", out("qk_vc", np.uint16), host_bf16(qvc).ravel()),
        ("padded norm output", out("pad", np.uint16), host_bf16(pout).ravel()),
        ("padded norm residual", out("pad_res", np.uint16), host_bf16(pres).ravel()),
        ("mla rope q (q_pe in place)", out("mr_q", np.uint16), host_bf16(mrq).ravel()),
        ("mla rope cache", out("mr_cache", np.uint16), host_bf16(mrc).ravel()),
    ]
    for what, c_side, py_side in pairs:
        assert c_side.shape == py_side.shape, (what, c_side.shape, py_side.shape)
        assert np.array_equal(c_side.view(np.uint8), py_side.view(np.uint8)), what
    # The calls did write: rotated q and the caches differ from their inputs.
    assert not np.array_equal(out("rope_q", np.uint16), rd["q"].ravel())
    assert not np.array_equal(out("rope_kc", np.uint16), rd["key_cache"].ravel())
    assert not np.array_equal(out("qk_qkv", np.uint16), qd["qkv"].ravel())
    assert not np.array_equal(out("mr_cache", np.uint16), rm["kv_cache"].ravel())
