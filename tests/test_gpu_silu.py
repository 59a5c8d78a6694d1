"""GPU parity: silu_mul_quant against the CPU oracle.

Covers the Llama-3-8B MLP workload (I = 14336, per-group 128, T in {1, 64,
1024, 8192}), group 64, static scale, a tensor-parallel shard width, ragged
widths, strided views and T = 0.  Every row is compared with the oracle at
every T; the amax-448 rule is checked on every group."""
import numpy as np
import pytest

import workloads
from gpu_util import (assert_codes, assert_scales, dev_bf16, host_f32, host_u8, require_gpu,
                      compare_rows, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rra():
    require_gpu()
    import rope_residual_add_amd as r

    r.lib()
    return r


def run(rra, oracle, T, I, mode, g=128, static=0.05, strided=False):
    import torch

    say(f"[silu] T={T} I={I} mode={mode} g={g} strided={strided}")
    d = workloads.silu_inputs(T, I)
    if strided:
        wide = np.zeros((T, 2 * I + 24), np.uint16)
        wide[:, 8:8 + 2 * I] = d["inp"]
        inp = dev_bf16(wide)[:, 8:8 + 2 * I]
        out = torch.empty((T, I + 8), dtype=torch.float8_e4m3fn, device="cuda")[:, :I]
    else:
        inp, out = dev_bf16(d["inp"]), None
    ss = torch.tensor([static], dtype=torch.float32, device="cuda") if mode == 1 else None
    out, scales = rra.silu_mul_quant(inp, mode, g if mode == 3 else 0, ss, out=out)
    torch.cuda.synchronize()
    rows = compare_rows(T)
    ref_codes, ref_scales = oracle.silu_mul_quant(d["inp"][rows], mode, g if mode == 3 else 0,
                                                  static)
    assert_codes(host_u8(out)[rows], ref_codes, f"codes T={T} I={I}")
    if mode == 3:
        assert_scales(host_f32(scales)[rows], ref_scales, "scales")
        if T:
            amax = out.float().abs().view(T, I // g, g).amax(dim=-1)
            assert torch.all((amax == 448.0) | (scales == 0))


@pytest.mark.parametrize("T", workloads.SILU.Ts)
def test_mlp_workload(rra, oracle, T):
    run(rra, oracle, T, workloads.SILU.I, 3, 128)


@pytest.mark.parametrize("T,I,mode,g", [(100, 14336, 3, 64), (64, 14336, 1, 0), (64, 1792, 3, 128),
                                        (33, 1000, 1, 0), (5, 64, 3, 64), (17, 2176, 3, 128)])
def test_shapes_and_modes(rra, oracle, T, I, mode, g):
    run(rra, oracle, T, I, mode, g)


def test_static_saturation(rra, oracle):
    """Static scale 1e-3: most codes saturate to +-448, none become NaN."""
    import torch

    say("[silu] static saturation")
    d = workloads.silu_inputs(5, 2048)
    ss = torch.tensor([1e-3], dtype=torch.float32, device="cuda")
    out, _ = rra.silu_mul_quant(dev_bf16(d["inp"]), 1, 0, ss)
    torch.cuda.synchronize()
    ref, _ = oracle.silu_mul_quant(d["inp"], 1, 0, 1e-3)
    codes = host_u8(out)
    assert_codes(codes, ref, "saturating codes")
    assert np.count_nonzero((codes & 0x7F) == 0x7E) > codes.size // 4
    assert not np.any((codes & 0x7F) == 0x7F)


def test_strided(rra, oracle):
    run(rra, oracle, 9, 2048, 3, 128, strided=True)


def test_empty(rra):
    import torch

    say("[silu] T=0")
    inp = torch.empty((0, 2048), dtype=torch.bfloat16, device="cuda")
    out, scales = rra.silu_mul_quant(inp, 3, 128)
    assert out.shape == (0, 1024) and scales.shape == (0, 8)
