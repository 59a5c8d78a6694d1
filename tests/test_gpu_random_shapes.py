"""GPU parity on seeded random shapes: every entry point against the oracle
over widths, head counts, head sizes, block sizes, strides, quant modes,
pairings, element types and padding drawn at random within the documented
limits (ragged widths that leave lanes and vectors partly used, one- and
many-pass tokens, T from 1 to a few hundred, and for the two norms a few
cases above their 1024-token switch of launch shape).  The cases are fixed by the
seed, so a failure names a reproducible shape.  Each case reuses the checks
of the op's own GPU test (codes within 1 ULP on at most 1e-4 of them, scales
and bf16/fp16 outputs within rtol 1e-2, caches exact outside the written
slots)."""
import dataclasses
import os

import numpy as np
import pytest

import workloads
from test_gpu_mla import run as run_dual
from test_gpu_next import run_mla_rope, run_pad, run_qknorm
from test_gpu_norm import run as run_norm
from test_gpu_rope import run as run_rope
from gpu_util import require_gpu
from test_gpu_silu import run as run_silu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rra():
    require_gpu()
    import rope_residual_add_amd as r

    r.lib()
    return r

# Cases per entry point; RRA_RANDOM_CASES widens a run (the first cases stay the same).
N_CASES = int(os.environ.get("RRA_RANDOM_CASES", "20"))
# RRA_RANDOM_SEED draws another family of cases (the default family is the one
# every run checks).
SEED = int(os.environ.get("RRA_RANDOM_SEED", "20261202"))


def _cases(tag, draw):
    rng = np.random.default_rng([SEED, sum(map(ord, tag))])  # fixed: the cases are stable
    return [draw(rng) for _ in range(N_CASES)]


def _mult(rng, lo, hi, m):
    """A random multiple of m in [lo, hi]."""
    return int(rng.integers(-(-lo // m), hi // m + 1)) * m


def _norm(rng):
    mode = int(rng.choice([1, 2, 3]))
    g = int(rng.choice([64, 128])) if mode == 3 else 0
    H = _mult(rng, g or 8, 8192, g or 8)
    return dict(T=int(rng.integers(1, 160)), H=H, mode=mode, g=g,
                eps=float(10 ** rng.uniform(-6, -2)), residual=bool(rng.integers(2)),
                strided=bool(rng.integers(2)))


def _silu(rng):
    mode = int(rng.choice([1, 3]))
    g = int(rng.choice([64, 128]))
    I = _mult(rng, g if mode == 3 else 8, 20000, g if mode == 3 else 8)
    return dict(T=int(rng.integers(1, 64)), I=I, mode=mode, g=g, strided=bool(rng.integers(2)))


def _rope(rng):
    D = int(rng.choice([64, 128, 256]))
    bs = int(rng.choice([1, 8, 16, 32]))
    T = int(rng.integers(1, 200))
    cfg = dataclasses.replace(workloads.ROPE, Hq=int(rng.integers(1, 72)), Hkv=int(rng.integers(1, 12)),
                              D=D, rot_dim=D, block_size=bs, num_blocks=-(-(T + 37) // bs),
                              max_pos=int(rng.integers(1, 4096)), is_neox=bool(rng.integers(2)),
                              dtype=str(rng.choice(["bf16", "f16"])))
    return dict(T=T, cfg=cfg, pad_every=int(rng.choice([0, 3, 7])), inplace=bool(rng.integers(2)),
                fused_qkv=bool(rng.integers(2)))


def _dual(rng):
    mode = int(rng.choice([0, 2, 3]))
    g = int(rng.choice([64, 128])) if mode == 3 else 0
    return dict(T=int(rng.integers(1, 160)), mode=mode, g=g, Hq=_mult(rng, g or 8, 2048, g or 8),
                Hkv=_mult(rng, 8, 1024, 8), eps_q=float(10 ** rng.uniform(-6, -2)),
                eps_kv=float(10 ** rng.uniform(-6, -2)), split_views=bool(rng.integers(2)))


def _qknorm(rng):
    D = int(rng.choice([64, 128, 256]))
    bs = int(rng.choice([1, 16, 32]))
    T = int(rng.integers(1, 160))
    cfg = dataclasses.replace(workloads.QKNORM, Hq=int(rng.integers(1, 72)),
                              Hkv=int(rng.integers(1, 12)), D=D, block_size=bs,
                              num_blocks=-(-(T + 11) // bs), max_pos=int(rng.integers(1, 4096)),
                              eps=float(10 ** rng.uniform(-6, -3)))
    cache = bool(rng.integers(2))
    return dict(T=T, cfg=cfg, cache=cache, write_k=bool(rng.integers(2)) or not cache,
                is_neox=bool(rng.integers(2)), pad_every=int(rng.choice([0, 4])) if cache else 0)


def _pad(rng):
    H = _mult(rng, 8, 8192, 8)
    return dict(T=int(rng.integers(1, 160)), H=H, H_pad=H + _mult(rng, 0, 512, 8),
                residual=bool(rng.integers(2)), eps=float(10 ** rng.uniform(-6, -2)),
                dtype=str(rng.choice(["bf16", "f16"])))


def _mla_rope(rng):
    rope = int(rng.choice([64, 128]))
    bs = int(rng.choice([1, 16, 64]))
    T = int(rng.integers(1, 120))
    cfg = dataclasses.replace(workloads.MLA_ROPE, Hq=int(rng.integers(1, 160)),
                              nope=_mult(rng, 0, 192, 8), rope_dim=rope,
                              kv_lora=_mult(rng, 8, 640, 8), is_neox=bool(rng.integers(2)),
                              block_size=bs, num_blocks=-(-(T + 5) // bs),
                              max_pos=int(rng.integers(1, 4096)))
    return dict(T=T, cfg=cfg, pad_every=int(rng.choice([0, 5])))


# The norms switch launch shape above 1024 rows (tokens): a few cases each
# above the switch, so that ragged widths reach the wide-row shapes too.
N_LARGE = max(1, N_CASES // 4)


def _large(draw):
    def f(rng):
        c = draw(rng)
        c["T"] = int(rng.integers(1025, 1400))
        return c
    return f


def _cases_large(tag, draw):
    rng = np.random.default_rng([20261202, sum(map(ord, tag)), 1])
    return [_large(draw)(rng) for _ in range(N_LARGE)]


@pytest.mark.parametrize("c", _cases("norm", _norm), ids=lambda c: f"T{c['T']}-H{c['H']}-m{c['mode']}")
def test_norm_random(rra, oracle, c):
    run_norm(rra, oracle, c["T"], c["H"], c["mode"], c["g"], eps=c["eps"],
             residual=c["residual"], strided=c["strided"])


@pytest.mark.parametrize("c", _cases("silu", _silu), ids=lambda c: f"T{c['T']}-I{c['I']}-m{c['mode']}")
def test_silu_random(rra, oracle, c):
    run_silu(rra, oracle, c["T"], c["I"], c["mode"], c["g"], strided=c["strided"])


@pytest.mark.parametrize("c", _cases("rope", _rope),
                         ids=lambda c: f"T{c['T']}-{c['cfg'].Hq}x{c['cfg'].Hkv}x{c['cfg'].D}")
def test_rope_random(rra, oracle, c):
    run_rope(rra, oracle, c["T"], c["cfg"], pad_every=c["pad_every"], inplace=c["inplace"],
             fused_qkv=c["fused_qkv"])


@pytest.mark.parametrize("c", _cases("dual", _dual), ids=lambda c: f"T{c['T']}-{c['Hq']}-{c['Hkv']}")
def test_dual_random(rra, oracle, c):
    run_dual(rra, oracle, c["T"], c["mode"], c["g"], c["eps_q"], c["eps_kv"], c["split_views"],
             Hq=c["Hq"], Hkv=c["Hkv"])


@pytest.mark.parametrize("c", _cases("qknorm", _qknorm),
                         ids=lambda c: f"T{c['T']}-{c['cfg'].Hq}x{c['cfg'].Hkv}x{c['cfg'].D}")
def test_qknorm_random(rra, oracle, c):
    run_qknorm(rra, oracle, c["T"], c["cfg"], cache=c["cache"], write_k=c["write_k"],
               is_neox=c["is_neox"], pad_every=c["pad_every"])


@pytest.mark.parametrize("c", _cases("pad", _pad), ids=lambda c: f"T{c['T']}-H{c['H']}-{c['H_pad']}")
def test_pad_random(rra, oracle, c):
    run_pad(rra, oracle, c["T"], c["H"], c["H_pad"], c["residual"], c["eps"], c["dtype"])


@pytest.mark.parametrize("c", _cases("mla_rope", _mla_rope),
                         ids=lambda c: f"T{c['T']}-{c['cfg'].Hq}x{c['cfg'].nope}+{c['cfg'].rope_dim}")
def test_mla_rope_random(rra, oracle, c):
    run_mla_rope(rra, oracle, c["T"], c["cfg"], pad_every=c["pad_every"])


@pytest.mark.parametrize("c", _cases_large("norm", _norm),
                         ids=lambda c: f"T{c['T']}-H{c['H']}-m{c['mode']}")
def test_norm_random_large_T(rra, oracle, c):
    run_norm(rra, oracle, c["T"], c["H"], c["mode"], c["g"], eps=c["eps"],
             residual=c["residual"], strided=c["strided"])


@pytest.mark.parametrize("c", _cases_large("dual", _dual), ids=lambda c: f"T{c['T']}-{c['Hq']}-{c['Hkv']}")
def test_dual_random_large_T(rra, oracle, c):
    run_dual(rra, oracle, c["T"], c["mode"], c["g"], c["eps_q"], c["eps_kv"], c["split_views"],
             Hq=c["Hq"], Hkv=c["Hkv"])
