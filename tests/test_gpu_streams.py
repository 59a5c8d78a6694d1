"""The binding launches on the caller's current stream.  Each call here runs on
a side stream right after that stream copies the real inputs into buffers that
held zeros, behind a spin kernel of several milliseconds: a launch on any other
stream would read the zeros.  Results are compared with the same calls made on
the default stream."""
import dataclasses

import numpy as np
import pytest

import workloads
from gpu_util import dev, dev_bf16, host_bf16, require_gpu, say

pytestmark = pytest.mark.gpu

SPIN_CYCLES = 20_000_000  # several milliseconds at the GPU's clock


@pytest.fixture(scope="module")
def rra():
    require_gpu()
    import rope_residual_add_amd as r

    r.lib()
    return r


def _on_side_stream(fill, call):
    """Zero-filled inputs; on a side stream: spin, fill, call.  Returns call's result."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch.cuda._sleep(SPIN_CYCLES)
        fill()
        out = call()
    side.synchronize()
    return out


def test_norm_and_silu_follow_the_current_stream(rra):
    import torch

    say("[streams] norm + silu on a side stream")
    n = workloads.norm_inputs(64, 4096)
    s = workloads.silu_inputs(64, 2048)
    src = dict(x=dev_bf16(n["x"]), res=dev_bf16(n["residual"]), inp=dev_bf16(s["inp"]))
    w = dev_bf16(n["weight"])
    ref_res = src["res"].clone()
    ref_codes, ref_scales = rra.fused_add_rmsnorm_quant(src["x"], ref_res, w, 1e-5, 2)
    ref_silu, ref_silu_s = rra.silu_mul_quant(src["inp"], 3, 128)
    torch.cuda.synchronize()

    buf = {k: torch.zeros_like(v) for k, v in src.items()}

    def fill():
        for k in buf:
            buf[k].copy_(src[k])

    def call():
        a = rra.fused_add_rmsnorm_quant(buf["x"], buf["res"], w, 1e-5, 2)
        b = rra.silu_mul_quant(buf["inp"], 3, 128)
        return a, b

    (codes, scales), (silu, silu_s) = _on_side_stream(fill, call)
    assert torch.equal(codes.view(torch.uint8), ref_codes.view(torch.uint8))
    assert torch.equal(scales, ref_scales)
    assert torch.equal(buf["res"].view(torch.int16), ref_res.view(torch.int16))
    assert torch.equal(silu.view(torch.uint8), ref_silu.view(torch.uint8))
    assert torch.equal(silu_s, ref_silu_s)


def test_rope_and_mla_norm_follow_the_current_stream(rra):
    import torch

    say("[streams] rope + MLA norm on a side stream")
    cfg = dataclasses.replace(workloads.ROPE, num_blocks=64)
    r = workloads.rope_inputs(48, cfg)
    m = workloads.mla_inputs(48)
    cs = rra.rope_cos_sin_cache(cfg.max_pos, cfg.rot_dim, cfg.theta)
    src = dict(q=dev_bf16(r["q"]), k=dev_bf16(r["k"]), v=dev_bf16(r["v"]),
               pos=dev(r["positions"]), slots=dev(r["slot_mapping"]), mq=dev_bf16(m["q"]),
               mkv=dev_bf16(m["kv"]))
    qw, kvw = dev_bf16(m["q_w"]), dev_bf16(m["kv_w"])
    kc0, vc0 = dev_bf16(r["key_cache"]), dev_bf16(r["value_cache"])

    ref_q, ref_kc, ref_vc = src["q"].clone(), kc0.clone(), vc0.clone()
    rra.rope_kv_write(src["pos"], ref_q, src["k"], src["v"], cs, src["slots"], ref_kc, ref_vc)
    ref_m = rra.dual_rmsnorm_quant(src["mq"], qw, 1e-6, src["mkv"], kvw, 1e-6, 3, 128)
    torch.cuda.synchronize()

    buf = {k: torch.zeros_like(v) for k, v in src.items()}
    # zero slots would all collide on slot 0: start from a distinct, wrong set instead
    buf["slots"].copy_(torch.arange(48, dtype=torch.int64, device="cuda") + 512)
    kc, vc = kc0.clone(), vc0.clone()

    def fill():
        for k in buf:
            buf[k].copy_(src[k])

    def call():
        rra.rope_kv_write(buf["pos"], buf["q"], buf["k"], buf["v"], cs, buf["slots"], kc, vc)
        return rra.dual_rmsnorm_quant(buf["mq"], qw, 1e-6, buf["mkv"], kvw, 1e-6, 3, 128)

    got_m = _on_side_stream(fill, call)
    assert np.array_equal(host_bf16(buf["q"]), host_bf16(ref_q))
    assert torch.equal(kc.view(torch.int16), ref_kc.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), ref_vc.view(torch.int16))
    for a, b in zip(got_m, ref_m):
        assert torch.equal(_bits(a), _bits(b))


def _bits(t):
    """The tensor's bit pattern, for exact comparison of FP8 / bf16 / fp32 data."""
    import torch

    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()])
