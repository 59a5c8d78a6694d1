"""GPU parity: dual_rmsnorm_quant (MLA q/kv latent norms in one launch) against
the CPU oracle.

Covers the DeepSeek-V3 shape (q latent 1536 with per-group-128 FP8 quant, kv
latent 512 kept bf16, eps 1e-6 for both; T in {1, 1024, 8192, 16384}), the
per-token and unquantized q variants, group 64, the two latents taken as
views of one [T, 1536 + 576] projection (kv = the first 512 columns of the
576-wide kv_a slice), distinct epsilons and T = 0.  Every row is compared
with the oracle at every T; the amax-448 rule is checked on every group."""
import numpy as np
import pytest

import workloads
from gpu_util import (assert_bf16, assert_codes, assert_scales, dev_bf16, host_bf16, host_f32,
                      host_u8, require_gpu, compare_rows, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rra():
    require_gpu()
    import rope_residual_add_amd as r

    r.lib()
    return r


def run(rra, oracle, T, mode=3, g=128, eps_q=1e-6, eps_kv=1e-6, split_views=False, Hq=1536,
        Hkv=512):
    import torch

    say(f"[mla] T={T} Hq={Hq} Hkv={Hkv} mode={mode} g={g} split_views={split_views}")
    cfg = workloads.MlaCfg("mla", Hq=Hq, Hkv=Hkv)
    d = workloads.mla_inputs(T, cfg)
    if split_views:
        # [T, q_lora | kv_lora | k_pe] as one projection output
        wide = np.zeros((T, Hq + Hkv + 64), np.uint16)
        wide[:, :Hq] = d["q"]
        wide[:, Hq:Hq + Hkv] = d["kv"]
        proj = dev_bf16(wide)
        q, kv = proj[:, :Hq], proj[:, Hq:Hq + Hkv]
    else:
        q, kv = dev_bf16(d["q"]), dev_bf16(d["kv"])
    qw, kvw = dev_bf16(d["q_w"]), dev_bf16(d["kv_w"])
    q_out, q_scales, kv_out = rra.dual_rmsnorm_quant(q, qw, eps_q, kv, kvw, eps_kv, mode,
                                                     g if mode == 3 else 0)
    torch.cuda.synchronize()

    rows = compare_rows(T)
    ref_q, ref_s, ref_kv = oracle.dual_rmsnorm_quant(d["q"][rows], d["q_w"], eps_q,
                                                     d["kv"][rows], d["kv_w"], eps_kv, mode,
                                                     g if mode == 3 else 0)
    if mode == 0:
        assert_bf16(host_bf16(q_out)[rows], ref_q, f"q_out T={T}")
    else:
        assert_codes(host_u8(q_out)[rows], ref_q, f"q codes T={T}", exact=True)
        assert_scales(host_f32(q_scales)[rows], ref_s, "q scales")
        if T:
            gg = Hq if mode == 2 else g
            amax = q_out.float().abs().view(T, Hq // gg, gg).amax(dim=-1)
            sc = q_scales.view(T, Hq // gg)
            assert torch.all((amax == 448.0) | (sc == 0))
    assert_bf16(host_bf16(kv_out)[rows], ref_kv, f"kv_out T={T}")


@pytest.mark.parametrize("T", workloads.MLA.Ts)
def test_mla_workload(rra, oracle, T):
    run(rra, oracle, T)


@pytest.mark.parametrize("mode,g", [(0, 0), (2, 0), (3, 64)])
def test_modes(rra, oracle, mode, g):
    run(rra, oracle, 37, mode, g)


# Up to 1024 tokens one wave per 512-column vector (four waves per token at
# the DeepSeek-V3 shape), above that one wave per token: both sides of the
# switch in every mode, and ragged widths on both paths.
@pytest.mark.parametrize("T", [1023, 1024, 1025])
@pytest.mark.parametrize("mode,g", [(0, 0), (2, 0), (3, 128), (3, 64)])
def test_decode_shape_switch(rra, oracle, T, mode, g):
    run(rra, oracle, T, mode, g)


@pytest.mark.parametrize("Hq,Hkv", [(1024, 512), (2048, 1024), (1000, 520), (512, 8)])
def test_decode_shape_widths(rra, oracle, Hq, Hkv):
    mode, g = (3, 64) if Hq % 64 == 0 else (2, 0)
    run(rra, oracle, 9, mode, g, Hq=Hq, Hkv=Hkv)
    run(rra, oracle, 1100, mode, g, Hq=Hq, Hkv=Hkv)


def test_split_views(rra, oracle):
    run(rra, oracle, 21, split_views=True)


def test_distinct_eps_and_widths(rra, oracle):
    run(rra, oracle, 9, eps_q=1e-2, eps_kv=1e-6)
    run(rra, oracle, 9, mode=2, Hq=2048, Hkv=1024)
    run(rra, oracle, 9, mode=3, g=64, Hq=192, Hkv=8)


def test_matches_per_token_norm(rra):
    """The q side in per-token mode is the plain RMSNorm + per-token quant of
    fused_add_rmsnorm_quant without a residual (same inputs, same codes)."""
    import torch

    say("[mla] q side == fused_add_rmsnorm_quant(residual=None)")
    d = workloads.mla_inputs(64)
    q, kv = dev_bf16(d["q"]), dev_bf16(d["kv"])
    qw, kvw = dev_bf16(d["q_w"]), dev_bf16(d["kv_w"])
    a_codes, a_scales, _ = rra.dual_rmsnorm_quant(q, qw, 1e-6, kv, kvw, 1e-6, 2)
    b_codes, b_scales = rra.fused_add_rmsnorm_quant(q, None, qw, 1e-6, 2)
    torch.cuda.synchronize()
    assert torch.equal(a_codes.view(torch.uint8), b_codes.view(torch.uint8))
    assert torch.equal(a_scales, b_scales)


def test_empty(rra):
    import torch

    say("[mla] T=0")
    e = lambda *s: torch.empty(s, dtype=torch.bfloat16, device="cuda")
    q_out, sc, kv_out = rra.dual_rmsnorm_quant(e(0, 1536), e(1536).fill_(1), 1e-6, e(0, 512),
                                               e(512).fill_(1), 1e-6, 3, 128)
    assert q_out.shape == (0, 1536) and sc.shape == (0, 12) and kv_out.shape == (0, 512)
