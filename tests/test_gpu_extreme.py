"""GPU parity on inputs of extreme magnitude and signed zeros.

The fast paths work in fp32; these cases push them out of its range, where
the kernels take their double-precision paths:
  * RMSNorm rows near the fp32 subnormal range (rho or 448 / amax beyond fp32,
    scales that are themselves subnormal), and rows near the bf16 maximum;
  * SiLU groups whose gates lie below about -88 (exp(-g) overflows fp32 and
    the fp32 activation flushes to zero), whose products g * u fall in the
    fp32 subnormal range, or that are all zero;
  * -0.0 inputs, whose code is 0x80 (e4m3fn keeps the sign of zero);
  * QK-norm heads whose mean square is below 2^-100 with eps = 0, or at or
    above 2^100 (where an fp32 sum of squares overflows);
  * SiLU groups whose products g * u exceed the fp32 range.
Bars as in the other parity tests (codes within one code on at most 1e-4 of
them, scales rtol 1e-2, bf16 within rtol 1e-2)."""
import numpy as np
import pytest

import workloads
from gpu_util import (assert_bf16, assert_codes, assert_scales, dev, dev_bf16, host_bf16,
                      host_f32, host_u8, require_gpu, say)
from helpers import bf16_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rra():
    require_gpu()
    import rope_residual_add_amd as r

    r.lib()
    return r


def _bf16(a) -> np.ndarray:
    return workloads.to_bf16_bits(np.asarray(a, np.float32))


NORM_ROWS = [  # (magnitude of x, eps)
    (1e-20, 0.0), (1e-30, 1e-6), (1e-38, 1e-5), (1e-39, 0.0), (1e36, 1e-6)]

# (T, H) reaching each launch shape of the residual-add norm: one vector per
# lane (T <= 1024), two vectors per lane, and three (H = 6144, where the codes
# of a dynamic scale are formed vector by vector rather than held).
NORM_SHAPES = [(64, 1024), (1100, 1024), (1030, 6144)]


@pytest.mark.parametrize("T,H", NORM_SHAPES)
@pytest.mark.parametrize("mode,g", [(1, 0), (2, 0), (3, 64), (3, 128)])
@pytest.mark.parametrize("mag,eps", NORM_ROWS)
def test_norm_extreme_rows(rra, oracle, mag, eps, mode, g, T, H):
    import torch

    say(f"[extreme] norm |x|~{mag:g} eps={eps:g} mode={mode} g={g} T={T} H={H}")
    rng = np.random.default_rng(11)
    x = _bf16(rng.standard_normal((T, H)) * mag)
    w = _bf16(1 + 0.1 * rng.standard_normal(H))
    static = 0.05
    ss = torch.tensor([static], dtype=torch.float32, device="cuda") if mode == 1 else None
    out, scales = rra.fused_add_rmsnorm_quant(dev_bf16(x), None, dev_bf16(w), eps, mode, g, ss)
    torch.cuda.synchronize()
    ref, ref_scales, _ = oracle.fused_add_rmsnorm_quant(x, None, w, eps, mode, g, static)
    assert_codes(host_u8(out), ref, f"codes |x|~{mag:g}", exact=True)
    if mode >= 2:
        assert_scales(host_f32(scales).reshape(ref_scales.shape), ref_scales, "scales")


def test_norm_negative_zero(rra, oracle):
    """Rows of ordinary values with -0.0 entries: their codes are 0x80 in every
    mode (zeros take the exact-quotient path)."""
    import torch

    say("[extreme] norm -0.0 entries")
    rng = np.random.default_rng(12)
    T, H = 32, 512
    x = _bf16(rng.standard_normal((T, H)))
    neg = rng.random((T, H)) < 0.1
    x[neg] = 0x8000
    w = _bf16(1 + 0.1 * rng.standard_normal(H))
    for mode, g in ((1, 0), (2, 0), (3, 64), (3, 128)):
        ss = torch.tensor([0.05], dtype=torch.float32, device="cuda") if mode == 1 else None
        out, _ = rra.fused_add_rmsnorm_quant(dev_bf16(x), None, dev_bf16(w), 1e-6, mode, g, ss)
        torch.cuda.synchronize()
        ref, _, _ = oracle.fused_add_rmsnorm_quant(x, None, w, 1e-6, mode, g, 0.05)
        codes = host_u8(out)
        assert (ref[neg] == 0x80).all()
        assert (codes[neg] == 0x80).all(), (mode, g, np.unique(codes[neg]))
        assert_codes(codes, ref, f"-0 codes mode={mode}", exact=True)


@pytest.mark.parametrize("T", [32, 1100])  # one wave per vector; one wave per token
@pytest.mark.parametrize("mag,eps", [(1e-20, 0.0), (1e-39, 0.0), (1e36, 1e-6)])
def test_dual_extreme_rows(rra, oracle, mag, eps, T):
    """MLA dual norm: bf16 kv output (rho beyond fp32 for the 1e-39 rows) and
    per-group FP8 q."""
    import torch

    say(f"[extreme] dual |x|~{mag:g} eps={eps:g} T={T}")
    rng = np.random.default_rng(13)
    Hq, Hkv = 1536, 512
    q = _bf16(rng.standard_normal((T, Hq)) * mag)
    kv = _bf16(rng.standard_normal((T, Hkv)) * mag)
    qw = _bf16(1 + 0.1 * rng.standard_normal(Hq))
    kw = _bf16(1 + 0.1 * rng.standard_normal(Hkv))
    q_out, q_sc, kv_out = rra.dual_rmsnorm_quant(dev_bf16(q), dev_bf16(qw), eps, dev_bf16(kv),
                                                 dev_bf16(kw), eps, 3, 128)
    torch.cuda.synchronize()
    rq, rs, rkv = oracle.dual_rmsnorm_quant(q, qw, eps, kv, kw, eps, 3, 128)
    assert_codes(host_u8(q_out), rq, "dual q codes", exact=True)
    assert_scales(host_f32(q_sc).reshape(rs.shape), rs, "dual q scales")
    assert_bf16(host_bf16(kv_out), rkv, "dual kv")


def test_silu_extreme_groups(rra, oracle):
    """Per-group SiLU with groups of gates in [-120, -90] and [-87, -80]
    (activations near or below the fp32 subnormal range), products of
    subnormal size, -0.0 gates, and an all-zero group."""
    import torch

    rng = np.random.default_rng(14)
    for G in (64, 128):
        say(f"[extreme] silu g={G}")
        T, I = 16, 6 * G
        g = rng.standard_normal((T, I)).astype(np.float32)
        u = rng.standard_normal((T, I)).astype(np.float32)
        g[:, 0:G] = rng.uniform(-120, -90, (T, G))
        g[:, G:2 * G] = rng.uniform(-87, -80, (T, G))
        u[:, 2 * G:3 * G] *= 1e-39
        g[:, 3 * G:4 * G] = 0.0
        u[:, 3 * G:4 * G] = 0.0
        g[:, 4 * G:5 * G][rng.random((T, G)) < 0.25] = -0.0
        inp = np.concatenate([_bf16(g), _bf16(u)], axis=1)
        out, sc = rra.silu_mul_quant(dev_bf16(inp), 3, G)
        torch.cuda.synchronize()
        ref, ref_scales = oracle.silu_mul_quant(inp, 3, G)
        codes, scales = host_u8(out), host_f32(sc)
        assert_codes(codes, ref, f"silu extreme codes g={G}")
        assert_scales(scales, ref_scales, f"silu extreme scales g={G}")
        assert (scales[:, 0:3] > 0).all() and (scales[:, 3] == 0).all()


def test_silu_products_beyond_fp32(rra, oracle):
    """Per-group SiLU where silu(g) * u exceeds fp32 (gates near 100, up values
    scaled by 2^120, and gates near -100 with huge up values, whose fp32
    product g * u would overflow before the sigmoid takes it back), plus one
    group whose amax / 448 exceeds fp32 (infinite scale, +-0 codes)."""
    import torch

    rng = np.random.default_rng(17)
    for G in (64, 128):
        say(f"[extreme] silu products beyond fp32 g={G}")
        T, I = 16, 4 * G
        g = (2.0 * rng.standard_normal((T, I))).astype(np.float32)
        u = rng.standard_normal((T, I)).astype(np.float32)
        g[:, :G] += 100.0
        u[:, :G] *= np.float32(2.0 ** 120)
        g[:, G:2 * G] -= 100.0
        u[:, G:2 * G] = rng.uniform(1e36, 3e38, (T, G)).astype(np.float32)
        g[0, 2 * G:3 * G] = 3e38
        u[0, 2 * G:3 * G] = 3e38
        inp = np.concatenate([_bf16(g), _bf16(u)], axis=1)
        out, sc = rra.silu_mul_quant(dev_bf16(inp), 3, G)
        torch.cuda.synchronize()
        ref, ref_scales = oracle.silu_mul_quant(inp, 3, G)
        codes, scales = host_u8(out), host_f32(sc)
        assert np.isinf(ref_scales[0, 2]) and np.isinf(scales[0, 2])
        assert_codes(codes, ref, f"silu beyond-fp32 codes g={G}")
        fin = np.isfinite(ref_scales)
        assert (np.isfinite(scales) == fin).all()
        assert_scales(np.where(fin, scales, 1.0), np.where(fin, ref_scales, 1.0),
                      f"silu beyond-fp32 scales g={G}")


@pytest.mark.parametrize("is_neox", [True, False])
def test_qknorm_tiny_heads(rra, oracle, is_neox):
    """QK norm with eps = 0 on heads of magnitude 1e-39 (bf16 subnormals) to
    1e-15, mixed with ordinary heads in the same token: the tiny heads are
    normalized from rescaled values, the others as usual (k written back)."""
    import dataclasses

    import torch

    say(f"[extreme] qknorm tiny heads neox={is_neox}")
    cfg = dataclasses.replace(workloads.QKNORM, eps=0.0)
    T, Hq, Hkv, D = 64, cfg.Hq, cfg.Hkv, cfg.D
    d = workloads.qknorm_inputs(T, cfg, with_cache=False)
    rng = np.random.default_rng(15)
    mags = np.array([1e-39, 1e-30, 1e-20, 1e-15, 1.0, 1e3])
    heads = Hq + Hkv
    x = rng.standard_normal((T, heads, D)) * mags[rng.integers(0, mags.size, (T, heads))][..., None]
    qkv = d["qkv"].copy()
    qkv[:, :heads * D] = _bf16(x.reshape(T, heads * D))
    g = dev_bf16(qkv)
    cs = rra.rope_cos_sin_cache(cfg.max_pos, D, cfg.theta)
    rra.qk_norm_rope_kv_write(dev(d["positions"]), g, dev_bf16(d["q_w"]), dev_bf16(d["k_w"]),
                              0.0, cs, Hq, Hkv, D, write_k=True, is_neox=is_neox)
    torch.cuda.synchronize()
    ref, _, _ = oracle.qk_norm_rope_kv_write(d["positions"], qkv, d["q_w"], d["k_w"], 0.0,
                                             cfg.theta, cfg.max_pos, Hq, Hkv, D, write_k=True,
                                             is_neox=is_neox)
    got = host_bf16(g)
    assert np.isfinite(bf16_to_f64(got[:, :heads * D])).all()
    assert_bf16(got[:, :heads * D], ref[:, :heads * D], "q and k, tiny heads")


@pytest.mark.parametrize("is_neox", [True, False])
def test_qknorm_large_heads(rra, oracle, is_neox):
    """QK norm (eps 1e-6) on heads of magnitude 1e18 to 1e37, among them 2^100,
    mixed with ordinary heads in the same token: an fp32 sum of squares of such
    a head overflows, so it is normalized from values scaled by 2^-100; the
    others as usual (k written back).  No output may be zero or non-finite."""
    import dataclasses

    import torch

    say(f"[extreme] qknorm large heads neox={is_neox}")
    cfg = dataclasses.replace(workloads.QKNORM, eps=1e-6)
    T, Hq, Hkv, D = 64, cfg.Hq, cfg.Hkv, cfg.D
    d = workloads.qknorm_inputs(T, cfg, with_cache=False)
    rng = np.random.default_rng(16)
    mags = np.array([1e18, 1e20, 2.0 ** 100, 1e36, 1e37, 1.0, 1e-3])
    heads = Hq + Hkv
    x = rng.standard_normal((T, heads, D)) * mags[rng.integers(0, mags.size, (T, heads))][..., None]
    qkv = d["qkv"].copy()
    qkv[:, :heads * D] = _bf16(x.reshape(T, heads * D))
    g = dev_bf16(qkv)
    cs = rra.rope_cos_sin_cache(cfg.max_pos, D, cfg.theta)
    rra.qk_norm_rope_kv_write(dev(d["positions"]), g, dev_bf16(d["q_w"]), dev_bf16(d["k_w"]),
                              cfg.eps, cs, Hq, Hkv, D, write_k=True, is_neox=is_neox)
    torch.cuda.synchronize()
    ref, _, _ = oracle.qk_norm_rope_kv_write(d["positions"], qkv, d["q_w"], d["k_w"], cfg.eps,
                                             cfg.theta, cfg.max_pos, Hq, Hkv, D, write_k=True,
                                             is_neox=is_neox)
    got = host_bf16(g)
    vals = bf16_to_f64(got[:, :heads * D]).reshape(T, heads, D)
    assert np.isfinite(vals).all()
    assert (np.abs(vals).max(axis=-1) > 0.1).all(), "a normalized head came out (near) zero"
    assert_bf16(got[:, :heads * D], ref[:, :heads * D], "q and k, large heads")


# ---- non-finite inputs -------------------------------------------------------
# NaN codes are compared as one class (0x7F and 0xFF, and for bf16 every NaN
# pattern): the sign of a NaN that arithmetic creates is not fixed by IEEE 754
# and differs between the host's and the GPU's arithmetic.

def _e4m3_nan_merged(c: np.ndarray) -> np.ndarray:
    c = c.copy()
    c[(c & 0x7F) == 0x7F] = 0x7F
    return c


def _bf16_nan_merged(h: np.ndarray) -> np.ndarray:
    h = h.copy()
    h[((h & 0x7F80) == 0x7F80) & ((h & 0x007F) != 0)] = 0x7FC0
    return h


def _special_norm_rows(rng, T, H):
    """Rows 1-5 hold a NaN, +inf, -inf, an all-zero row with -0.0 entries and
    an all -0.0 row; the rest are ordinary."""
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[1, 5] = np.nan
    x[2, 7] = np.inf
    x[3, 9] = -np.inf
    x[4] = 0.0
    x[4, ::3] = -0.0
    x[5] = -0.0
    return _bf16(x), [1, 2, 3, 4, 5]


@pytest.mark.parametrize("T,H", [(16, 1024), (1030, 6144)])
@pytest.mark.parametrize("mode,g", [(1, 0), (2, 0), (3, 64), (3, 128)])
def test_norm_non_finite_rows(rra, oracle, mode, g, T, H):
    """A row holding a NaN or an infinity: rho is NaN or 0, and the oracle's
    reading gives scale 0 and +0 codes for every dynamic slice of it (the amax
    of NaN values is 0), NaN codes (static scale) where a value is NaN.  Zero
    rows with -0.0 entries get scale 0 and +0 codes."""
    import torch

    say(f"[extreme] norm non-finite rows mode={mode} g={g} T={T} H={H}")
    rng = np.random.default_rng(16)
    x, special = _special_norm_rows(rng, T, H)
    w = _bf16(1 + 0.1 * rng.standard_normal(H))
    ss = torch.tensor([0.05], dtype=torch.float32, device="cuda") if mode == 1 else None
    out, scales = rra.fused_add_rmsnorm_quant(dev_bf16(x), None, dev_bf16(w), 1e-6, mode, g, ss)
    torch.cuda.synchronize()
    ref, ref_scales, _ = oracle.fused_add_rmsnorm_quant(x, None, w, 1e-6, mode, g, 0.05)
    codes = host_u8(out)
    ordinary = np.setdiff1d(np.arange(T), special)
    assert np.array_equal(_e4m3_nan_merged(codes[special]), _e4m3_nan_merged(ref[special]))
    assert_codes(codes[ordinary], ref[ordinary], "ordinary rows", exact=True)
    if mode >= 2:
        got = host_f32(scales).reshape(ref_scales.shape)
        assert not np.isnan(got).any()
        assert (got[special] == 0).all() and (ref_scales[special] == 0).all()
        assert_scales(got[ordinary], ref_scales[ordinary], "ordinary scales")


@pytest.mark.parametrize("T", [16, 1100])
def test_dual_non_finite_rows(rra, oracle, T):
    import torch

    say(f"[extreme] dual non-finite rows T={T}")
    rng = np.random.default_rng(17)
    Hq, Hkv = 1536, 512
    q, special = _special_norm_rows(rng, T, Hq)
    kv, _ = _special_norm_rows(rng, T, Hkv)
    qw = _bf16(1 + 0.1 * rng.standard_normal(Hq))
    kw = _bf16(1 + 0.1 * rng.standard_normal(Hkv))
    q_out, q_sc, kv_out = rra.dual_rmsnorm_quant(dev_bf16(q), dev_bf16(qw), 1e-6, dev_bf16(kv),
                                                 dev_bf16(kw), 1e-6, 3, 128)
    torch.cuda.synchronize()
    rq, rs, rkv = oracle.dual_rmsnorm_quant(q, qw, 1e-6, kv, kw, 1e-6, 3, 128)
    ordinary = np.setdiff1d(np.arange(T), special)
    codes, kvg, sc = host_u8(q_out), host_bf16(kv_out), host_f32(q_sc).reshape(rs.shape)
    assert np.array_equal(_e4m3_nan_merged(codes[special]), _e4m3_nan_merged(rq[special]))
    assert (sc[special] == 0).all() and (rs[special] == 0).all()
    assert np.array_equal(_bf16_nan_merged(kvg[special]), _bf16_nan_merged(rkv[special]))
    assert_codes(codes[ordinary], rq[ordinary], "dual ordinary q", exact=True)
    assert_bf16(kvg[ordinary], rkv[ordinary], "dual ordinary kv")


@pytest.mark.parametrize("mode,G", [(1, 0), (3, 64), (3, 128)])
def test_silu_non_finite(rra, oracle, mode, G):
    """NaN and infinite gates and ups: NaN activations code as NaN and do not
    count towards a group's amax; an infinite activation makes the group's
    scale infinite (its other codes +-0); a group of -0.0 products gets scale 0
    and +0 codes; a static scale saturates infinities and keeps NaN."""
    import torch

    say(f"[extreme] silu non-finite mode={mode} g={G}")
    rng = np.random.default_rng(18)
    T, I = 8, 512
    g = (2 * rng.standard_normal((T, I))).astype(np.float32)
    u = rng.standard_normal((T, I)).astype(np.float32)
    g[1, 5] = np.nan
    g[2, 7] = np.inf
    g[3, 9] = -np.inf
    u[4, 10] = np.inf
    u[5, 11] = np.nan
    g[6, :128] = -0.0
    special = (np.isnan(g) | np.isinf(g) | np.isnan(u) | np.isinf(u))
    special[6, :128] = True
    inp = np.concatenate([_bf16(g), _bf16(u)], axis=1)
    ss = torch.tensor([0.05], dtype=torch.float32, device="cuda") if mode == 1 else None
    out, sc = rra.silu_mul_quant(dev_bf16(inp), mode, G, ss)
    torch.cuda.synchronize()
    ref, ref_scales = oracle.silu_mul_quant(inp, mode, G, 0.05)
    codes = host_u8(out)
    assert np.array_equal(_e4m3_nan_merged(codes[special]), _e4m3_nan_merged(ref[special]))
    assert_codes(np.where(special, 0, codes), np.where(special, 0, ref).astype(np.uint8),
                 "silu other codes")
    if mode == 3:
        got = host_f32(sc)
        assert not np.isnan(got).any()
        assert_scales(got, ref_scales, "silu scales")
