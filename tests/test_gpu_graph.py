"""The entry points allocate nothing and never synchronize, so a caller can
capture them into a HIP graph (torch.cuda.CUDAGraph) and replay it.  This test
captures one pass of the four fused kernels, replays it several times with new
inputs copied into the captured buffers between replays (eager work and
synchronizations in between), and checks every replay bit-for-bit against the
same calls made eagerly."""
import pytest

import workloads
from gpu_util import dev, dev_bf16, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rra():
    require_gpu()
    import rope_residual_add_amd as r

    r.lib()
    return r


# T = 96 runs the norms' decode-size launch shapes, T = 1100 their wider ones.
@pytest.mark.parametrize("T,num_blocks", [(96, 64), (1100, 128)])
def test_graph_replays_match_eager(rra, T, num_blocks):
    import dataclasses

    import torch

    say(f"[graph] capture four kernels at T={T}, replay with fresh inputs")
    rcfg = dataclasses.replace(workloads.ROPE, num_blocks=num_blocks)

    def load(salt):
        """Host inputs for one replay (seeded by salt)."""
        n = workloads.norm_inputs(T, 4096, salt=salt)
        s = workloads.silu_inputs(T, 2048, salt=salt)
        r = workloads.rope_inputs(T, rcfg, salt=salt)
        m = workloads.mla_inputs(T, salt=salt)
        return n, s, r, m

    def to_device(host):
        n, s, r, m = host
        return dict(x=dev_bf16(n["x"]), res=dev_bf16(n["residual"]), w=dev_bf16(n["weight"]),
                    inp=dev_bf16(s["inp"]), q=dev_bf16(r["q"]), k=dev_bf16(r["k"]),
                    v=dev_bf16(r["v"]), pos=dev(r["positions"]), slots=dev(r["slot_mapping"]),
                    kc=dev_bf16(r["key_cache"]), vc=dev_bf16(r["value_cache"]),
                    mq=dev_bf16(m["q"]), mkv=dev_bf16(m["kv"]), mqw=dev_bf16(m["q_w"]),
                    mkvw=dev_bf16(m["kv_w"]))

    cs = rra.rope_cos_sin_cache(rcfg.max_pos, rcfg.rot_dim, rcfg.theta)
    outs = dict(
        norm=torch.empty((T, 4096), dtype=torch.float8_e4m3fn, device="cuda"),
        norm_s=torch.empty((T,), dtype=torch.float32, device="cuda"),
        silu=torch.empty((T, 2048), dtype=torch.float8_e4m3fn, device="cuda"),
        silu_s=torch.empty((T, 16), dtype=torch.float32, device="cuda"),
        mq=torch.empty((T, 1536), dtype=torch.float8_e4m3fn, device="cuda"),
        mq_s=torch.empty((T, 12), dtype=torch.float32, device="cuda"),
        mkv=torch.empty((T, 512), dtype=torch.bfloat16, device="cuda"),
    )

    def step(b):
        rra.fused_add_rmsnorm_quant(b["x"], b["res"], b["w"], 1e-5, "per_token", 0, None,
                                    outs["norm"], outs["norm_s"])
        rra.silu_mul_quant(b["inp"], "per_group", 128, None, outs["silu"], outs["silu_s"])
        rra.rope_kv_write(b["pos"], b["q"], b["k"], b["v"], cs, b["slots"], b["kc"], b["vc"])
        rra.dual_rmsnorm_quant(b["mq"], b["mqw"], 1e-6, b["mkv"], b["mkvw"], 1e-6, "per_group",
                               128, outs["mq"], outs["mq_s"], outs["mkv"])

    def snapshot(b):
        keys = ("res", "q", "kc", "vc")
        vals = {k: b[k].clone() for k in keys}
        vals.update({k: v.clone() for k, v in outs.items()})
        return vals

    # captured buffers
    bufs = to_device(load(0))
    step(bufs)  # warm-up outside the graph
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            step(bufs)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()

    for salt in (1, 2, 3):
        host = load(salt)
        # eager reference on fresh buffers
        ref_bufs = to_device(host)
        step(ref_bufs)
        torch.cuda.synchronize()
        ref = snapshot(ref_bufs)
        # the same inputs copied into the captured buffers, then one replay
        fresh = to_device(host)
        for k, t in fresh.items():
            bufs[k].copy_(t)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot(bufs)
        for k in ref:
            a, b = ref[k], got[k]
            if a.dtype in (torch.float8_e4m3fn, torch.bfloat16):
                a, b = a.view(torch.uint8), b.view(torch.uint8)
            assert torch.equal(a, b), f"replay {salt}: {k} differs from eager"
        print(f"replay {salt}: all outputs bit-identical to eager", flush=True)
