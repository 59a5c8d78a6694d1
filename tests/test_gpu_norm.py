"""GPU parity: fused_add_rmsnorm_quant against the CPU oracle.

Covers the static-scale workload (H=1024, eps 1e-6, scale 0.05, T in {16,
8192}), the per-token workload (Llama-3-8B width 4096, eps 1e-5, T in {1, 32,
512, 8192}), per-group 128/64, no residual, ragged widths that leave masked
lanes, strided views and T = 0.  Every row is compared with the oracle at
every T, and properties that hold at any size (residual = bf16(x + residual),
a row amax of exactly 448) are checked as well."""
import numpy as np
import pytest

import workloads
from helpers import TIE_CASES
from gpu_util import (assert_codes, assert_scales, dev_bf16, host_bf16, host_f32, host_u8,
                      require_gpu, compare_rows, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rra():
    require_gpu()
    import rope_residual_add_amd as r

    r.lib()
    return r


def _strided(a: np.ndarray, pad_left: int, pad_right: int):
    """Device bf16 view [T, H] inside a wider [T, pad_left + H + pad_right] buffer."""
    T, H = a.shape
    wide = np.zeros((T, pad_left + H + pad_right), np.uint16)
    wide[:, pad_left:pad_left + H] = a
    return dev_bf16(wide)[:, pad_left:pad_left + H]


def run(rra, oracle, T, H, mode, g=0, eps=1e-5, static=0.05, residual=True, tag="norm_token",
        strided=False):
    import torch

    say(f"[norm] T={T} H={H} mode={mode} g={g} residual={residual} strided={strided}")
    d = workloads.norm_inputs(T, H, tag=tag)
    if strided:
        x = _strided(d["x"], 32, 40)
        r = _strided(d["residual"], 8, 0) if residual else None
        out_wide = torch.empty((T, H + 16), dtype=torch.float8_e4m3fn, device="cuda")
        out = out_wide[:, 8:8 + H]
    else:
        x = dev_bf16(d["x"])
        r = dev_bf16(d["residual"]) if residual else None
        out = None
    r_before = r.clone() if residual else None
    w = dev_bf16(d["weight"])
    ss = torch.tensor([static], dtype=torch.float32, device="cuda") if mode == 1 else None
    out, scales = rra.fused_add_rmsnorm_quant(x, r, w, eps, mode, g, ss, out=out)
    torch.cuda.synchronize()

    rows = compare_rows(T)
    ref_codes, ref_scales, ref_res = oracle.fused_add_rmsnorm_quant(
        d["x"][rows], d["residual"][rows] if residual else None, d["weight"], eps, mode, g, static)
    assert_codes(host_u8(out)[rows], ref_codes, f"codes T={T} H={H} mode={mode}", exact=True)
    if scales is not None:
        assert_scales(host_f32(scales)[rows], ref_scales, "scales")
    if residual:
        assert np.array_equal(host_bf16(r)[rows], ref_res)
        # any size: the stored residual is bf16(x + old residual) on every row
        full = (x.float() + r_before.float()).to(torch.bfloat16)
        assert torch.equal(full.view(torch.int16), r.view(torch.int16))
    if mode == 2 and T:
        # any size: every row reaches the largest code
        amax = out.float().abs().amax(dim=1)
        assert torch.all(amax == 448.0)
    return out, scales


@pytest.mark.parametrize("T", workloads.NORM_STATIC.Ts)
def test_static_workload(rra, oracle, T):
    c = workloads.NORM_STATIC
    run(rra, oracle, T, c.H, 1, eps=c.eps, static=c.static_scale, tag="norm_static")


@pytest.mark.parametrize("T", workloads.NORM_TOKEN.Ts)
def test_per_token_workload(rra, oracle, T):
    c = workloads.NORM_TOKEN
    run(rra, oracle, T, c.H, 2, eps=c.eps)


@pytest.mark.parametrize("T,g", [(7, 128), (8192, 128), (33, 64), (512, 64)])
def test_per_group(rra, oracle, T, g):
    run(rra, oracle, T, 4096, 3, g)


# Up to 1024 rows the kernel runs one vector per lane (a row over up to 16
# waves), above that four waves per row with two vectors per lane (H = 4096):
# both sides of the switch, every mode, and widths of 1 to 16 waves per row.
@pytest.mark.parametrize("T", [1023, 1024, 1025])
@pytest.mark.parametrize("mode,g", [(1, 0), (2, 0), (3, 128), (3, 64)])
def test_decode_shape_switch(rra, oracle, T, mode, g):
    run(rra, oracle, T, 4096, mode, g)


@pytest.mark.parametrize("H", [512, 1024, 2048, 3072, 6144, 8192])
def test_decode_shape_widths(rra, oracle, H):
    run(rra, oracle, 24, H, 3, 64)
    run(rra, oracle, 1100, H, 2)


@pytest.mark.parametrize("mode,g", [(1, 0), (2, 0), (3, 128)])
def test_no_residual(rra, oracle, mode, g):
    run(rra, oracle, 33, 4096, mode, g, residual=False)


@pytest.mark.parametrize("H,mode,g", [(8, 2, 0), (1000, 1, 0), (2880, 2, 0), (2880, 3, 64),
                                      (5120, 3, 128), (8192, 2, 0), (7168, 3, 128)])
def test_widths(rra, oracle, H, mode, g):
    run(rra, oracle, 65, H, mode, g)


@pytest.mark.parametrize("T,H,mode,g", [(33, 1536, 2, 0), (7, 2048, 3, 128), (3, 1024, 2, 0),
                                        (1, 2048, 1, 0), (2, 8192, 3, 64)])
def test_ragged_row_blocks(rra, oracle, T, H, mode, g):
    """Token counts that leave rows of the last workgroup unused, for each
    number of waves per row (1, 2 and 4)."""
    run(rra, oracle, T, H, mode, g)


@pytest.mark.parametrize("mode,g", [(2, 0), (3, 128), (1, 0)])
def test_strided_views(rra, oracle, mode, g):
    run(rra, oracle, 19, 1024, mode, g, strided=True)


def test_static_saturation(rra, oracle):
    """A static scale far below amax / 448 drives most |y| / s past 448: those
    codes saturate to +-448 (0x7E / 0xFE), never NaN (0x7F / 0xFF)."""
    out, _ = run(rra, oracle, 9, 4096, 1, static=1e-3)
    codes = host_u8(out)
    assert np.count_nonzero((codes & 0x7F) == 0x7E) > codes.size // 4
    assert not np.any((codes & 0x7F) == 0x7F)


def test_empty(rra):
    import torch

    say("[norm] T=0")
    x = torch.empty((0, 1024), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(1024, dtype=torch.bfloat16, device="cuda")
    out, scales = rra.fused_add_rmsnorm_quant(x, x.clone(), w, 1e-6, 2)
    assert out.shape == (0, 1024) and scales.shape == (0,)


def test_zero_rows(rra):
    """An all-zero row gets scale 0 and all-zero codes (no NaN)."""
    import torch

    say("[norm] zero rows")
    x = torch.zeros((8, 512), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(512, dtype=torch.bfloat16, device="cuda")
    for mode, g in ((2, 0), (3, 64)):
        out, scales = rra.fused_add_rmsnorm_quant(x, None, w, 1e-6, mode, g)
        torch.cuda.synchronize()
        assert torch.all(scales == 0)
        assert torch.all((out.view(torch.uint8) & 0x7F) == 0)


def test_error_is_raised(rra):
    import torch

    x = torch.zeros((4, 1000), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(1000, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rra.RRAError):
        rra.fused_add_rmsnorm_quant(x, None, w, 1e-6, 3, 128)


@pytest.mark.parametrize("s,m,z0,w0,eps,code,side", TIE_CASES)
def test_exact_tie_rounds_to_even(rra, s, m, z0, w0, eps, code, side):
    """Rows built so that y / s is exactly an e4m3 midpoint (rho = 1, y = z0 *
    w0, static scale s): the code must be the even one, bit for bit, here as
    in the oracle's pin.  Nine rows of 1024, one launch (several workgroups,
    and the same row at every T position)."""
    import torch

    say(f"[norm] exact tie m={m} s={s}")
    H, T = 8, 1024
    x = torch.zeros((T, H), dtype=torch.float32)
    x[:, 0] = z0
    w = torch.ones(H, dtype=torch.float32)
    w[0] = w0
    x, w = x.to(torch.bfloat16).cuda(), w.to(torch.bfloat16).cuda()
    ss = torch.tensor([s], dtype=torch.float32, device="cuda")
    out, _ = rra.fused_add_rmsnorm_quant(x, None, w, eps, 1, 0, ss)
    torch.cuda.synchronize()
    got = out.view(torch.uint8).cpu().numpy()
    assert (got[:, 0] == code).all() and not got[:, 1:].any(), (got[:, 0][:4], code)
