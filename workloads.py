"""Seeded synthetic inputs for the four fused kernels.

Shared by the tests, the benchmark and the smoke check, and by both the HIP
path and the CPU oracle.  It holds none of the method's arithmetic: it only
draws random numbers (numpy ``default_rng``) and stores them as bf16 bit
patterns (torch's float32 -> bfloat16 conversion, round-to-nearest-even) or,
for the fp16 variants, IEEE fp16 bit patterns (numpy's float32 -> float16
conversion, round-to-nearest-even).

Layer shapes are those of Llama-3-8B (hidden 4096, intermediate 14336, 32 query
/ 8 key-value heads of 128, rope theta 500000) and of DeepSeek-V3's MLA
(q_lora_rank 1536, kv_lora_rank 512).  No weights or datasets are involved.

Seeding: every tensor comes from ``default_rng((tag, T, index, salt))`` where
``tag`` names the workload, ``T`` is the token count, ``index`` numbers the
tensor within the workload and ``salt`` lets callers draw independent copies
(the benchmark's rotating buffer sets).
"""
from __future__ import annotations

import dataclasses

import numpy as np

_TAGS = {"norm_static": 0, "norm_token": 1, "silu": 2, "rope": 3, "mla": 4,
         "qknorm": 5, "pad": 6, "mla_rope": 7}


@dataclasses.dataclass(frozen=True)
class NormCfg:
    """Residual add + RMSNorm + FP8 quant."""
    name: str
    H: int
    eps: float
    quant: str  # "static" | "per_token" | "per_group"
    group_size: int = 0
    static_scale: float = 0.05
    Ts: tuple = ()


@dataclasses.dataclass(frozen=True)
class SiluCfg:
    """SiLU-and-Mul + FP8 quant."""
    name: str
    I: int
    quant: str
    group_size: int = 128
    static_scale: float = 0.05
    Ts: tuple = ()


@dataclasses.dataclass(frozen=True)
class RopeCfg:
    """Neox RoPE + paged KV-cache write."""
    name: str
    Hq: int = 32
    Hkv: int = 8
    D: int = 128
    rot_dim: int = 128
    theta: float = 500000.0
    max_pos: int = 8192
    num_blocks: int = 4096
    block_size: int = 16
    is_neox: bool = True
    Ts: tuple = ()
    dtype: str = "bf16"  # element type of q, k, v and the caches: "bf16" or "f16"


@dataclasses.dataclass(frozen=True)
class MlaCfg:
    """MLA dual RMSNorm with per-group FP8 quant of the q latent."""
    name: str
    Hq: int = 1536
    Hkv: int = 512
    eps_q: float = 1e-6
    eps_kv: float = 1e-6
    quant: str = "per_group"
    group_size: int = 128
    Ts: tuple = ()


# The five workloads and their token-count sets; T = 8192 is the headline
# point for every kernel.
NORM_STATIC = NormCfg("norm_static", H=1024, eps=1e-6, quant="static", static_scale=0.05,
                      Ts=(16, 8192))
NORM_TOKEN = NormCfg("norm_token", H=4096, eps=1e-5, quant="per_token", Ts=(1, 32, 512, 8192))
SILU = SiluCfg("silu", I=14336, quant="per_group", group_size=128, Ts=(1, 64, 1024, 8192))
ROPE = RopeCfg("rope", Ts=(16, 2048, 8192, 16384))
ROPE_F16 = RopeCfg("rope_f16", Ts=(16, 2048, 8192), dtype="f16")
MLA = MlaCfg("mla", Ts=(1, 1024, 8192, 16384))

HEADLINE_T = 8192


@dataclasses.dataclass(frozen=True)
class QkNormCfg:
    """Per-head QK RMSNorm + RoPE + paged KV write (Qwen3-8B attention shape)."""
    name: str = "qknorm"
    Hq: int = 32
    Hkv: int = 8
    D: int = 128
    eps: float = 1e-6
    theta: float = 1000000.0
    max_pos: int = 8192
    num_blocks: int = 4096
    block_size: int = 16
    Ts: tuple = (16, 2048, 8192)


@dataclasses.dataclass(frozen=True)
class PadCfg:
    """Residual add + RMSNorm + padding (GPT-OSS hidden 2880 -> 3072)."""
    name: str = "pad"
    H: int = 2880
    H_pad: int = 3072
    eps: float = 1e-5
    Ts: tuple = (16, 2048, 8192)
    dtype: str = "bf16"  # element type of x, residual, weight and out: "bf16" or "f16"


@dataclasses.dataclass(frozen=True)
class MlaRopeCfg:
    """MLA q_pe / k_pe RoPE + [kv_c | k_pe] cache write (DeepSeek-V3: 128
    heads of nope 128 + rope 64, kv_lora 512, GPT-J pairing)."""
    name: str = "mla_rope"
    Hq: int = 128
    nope: int = 128
    rope_dim: int = 64
    kv_lora: int = 512
    theta: float = 10000.0
    max_pos: int = 8192
    num_blocks: int = 1024
    block_size: int = 64
    is_neox: bool = False
    Ts: tuple = (16, 2048, 8192)


QKNORM = QkNormCfg()
PAD = PadCfg()
PAD_F16 = PadCfg(name="pad_f16", dtype="f16")
MLA_ROPE = MlaRopeCfg()


def _rng(tag: str, T: int, index: int, salt: int = 0) -> np.random.Generator:
    return np.random.default_rng((_TAGS[tag], int(T), int(index), int(salt)))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even, via torch."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_normal(rng: np.random.Generator, shape, mean: float = 0.0, std: float = 1.0):
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return to_bf16_bits(a)


def f16_normal(rng: np.random.Generator, shape):
    """N(0, 1) draws as IEEE fp16 bit patterns (numpy's round-to-nearest-even)."""
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16).view(np.uint16)


def elem_normal(dtype: str, rng: np.random.Generator, shape):
    return f16_normal(rng, shape) if dtype == "f16" else bf16_normal(rng, shape)


def norm_inputs(T: int, H: int, salt: int = 0, tag: str = "norm_token", dtype: str = "bf16"):
    """x, residual ~ N(0,1) [T,H]; weight ~ N(1, 0.1) [H]; bit patterns of dtype."""
    if dtype == "f16":
        w = 1.0 + 0.1 * _rng(tag, 0, 2, salt).standard_normal(H, dtype=np.float32)
        return dict(x=f16_normal(_rng(tag, T, 0, salt), (T, H)),
                    residual=f16_normal(_rng(tag, T, 1, salt), (T, H)),
                    weight=w.astype(np.float16).view(np.uint16))
    return dict(
        x=bf16_normal(_rng(tag, T, 0, salt), (T, H)),
        residual=bf16_normal(_rng(tag, T, 1, salt), (T, H)),
        weight=bf16_normal(_rng(tag, 0, 2, salt), (H,), mean=1.0, std=0.1),
    )


def silu_inputs(T: int, I: int, salt: int = 0):
    """gate | up halves of one [T, 2I] row block, ~ N(0, 2) (std 2)."""
    return dict(inp=bf16_normal(_rng("silu", T, 0, salt), (T, 2 * I), std=2.0))


def rope_inputs(T: int, cfg: RopeCfg = ROPE, salt: int = 0, with_cache: bool = True):
    """q [T,Hq,D], k, v [T,Hkv,D] ~ N(0,1) as cfg.dtype bit patterns; positions
    uniform in [0, max_pos); slot_mapping = the first T entries of a seeded
    permutation of all cache slots (distinct); caches filled with a seeded
    random sentinel pattern (finite in bf16 and in fp16)."""
    n_slots = cfg.num_blocks * cfg.block_size
    if T > n_slots:
        raise ValueError("more tokens than cache slots")
    d = dict(
        q=elem_normal(cfg.dtype, _rng("rope", T, 0, salt), (T, cfg.Hq, cfg.D)),
        k=elem_normal(cfg.dtype, _rng("rope", T, 1, salt), (T, cfg.Hkv, cfg.D)),
        v=elem_normal(cfg.dtype, _rng("rope", T, 2, salt), (T, cfg.Hkv, cfg.D)),
        positions=_rng("rope", T, 3, salt).integers(0, cfg.max_pos, T, dtype=np.int64),
        slot_mapping=_rng("rope", T, 4, salt).permutation(n_slots)[:T].astype(np.int64),
    )
    if with_cache:
        shape = (cfg.num_blocks, cfg.block_size, cfg.Hkv, cfg.D)
        d["key_cache"] = sentinel_cache(shape, 5, salt)
        d["value_cache"] = sentinel_cache(shape, 6, salt)
    return d


def sentinel_cache(shape, index: int, salt: int = 0) -> np.ndarray:
    """Random 16-bit patterns with bit 14 clear, so the exponent field is below
    all-ones and the value finite whether read as bf16 or as fp16."""
    r = _rng("rope", 0, index, salt).integers(0, 1 << 16, size=shape, dtype=np.uint16)
    return (r & np.uint16(0xBFFF)).astype(np.uint16)  # clear the top exponent bit


def qknorm_inputs(T: int, cfg: QkNormCfg = QKNORM, salt: int = 0, with_cache: bool = True):
    """qkv [T, (Hq + 2 Hkv) D] ~ N(0,1); q and k norm weights ~ N(1, 0.1) of D;
    positions uniform in [0, max_pos); distinct slots; sentinel caches."""
    n_slots = cfg.num_blocks * cfg.block_size
    if T > n_slots:
        raise ValueError("more tokens than cache slots")
    d = dict(
        qkv=bf16_normal(_rng("qknorm", T, 0, salt), (T, (cfg.Hq + 2 * cfg.Hkv) * cfg.D)),
        q_w=bf16_normal(_rng("qknorm", 0, 1, salt), (cfg.D,), mean=1.0, std=0.1),
        k_w=bf16_normal(_rng("qknorm", 0, 2, salt), (cfg.D,), mean=1.0, std=0.1),
        positions=_rng("qknorm", T, 3, salt).integers(0, cfg.max_pos, T, dtype=np.int64),
        slot_mapping=_rng("qknorm", T, 4, salt).permutation(n_slots)[:T].astype(np.int64),
    )
    if with_cache:
        shape = (cfg.num_blocks, cfg.block_size, cfg.Hkv, cfg.D)
        d["key_cache"] = sentinel_cache(shape, 5, salt)
        d["value_cache"] = sentinel_cache(shape, 6, salt)
    return d


def pad_inputs(T: int, cfg: PadCfg = PAD, salt: int = 0):
    """x, residual ~ N(0,1) [T, H]; weight ~ N(1, 0.1)."""
    return norm_inputs(T, cfg.H, salt=salt, tag="pad", dtype=cfg.dtype)


def mla_rope_inputs(T: int, cfg: MlaRopeCfg = MLA_ROPE, salt: int = 0, with_cache: bool = True):
    """q [T, Hq * (nope + rope_dim)], k_pe [T, rope_dim], kv_c [T, kv_lora]
    ~ N(0,1); positions uniform; distinct slots; a sentinel cache."""
    n_slots = cfg.num_blocks * cfg.block_size
    if T > n_slots:
        raise ValueError("more tokens than cache slots")
    d = dict(
        q=bf16_normal(_rng("mla_rope", T, 0, salt), (T, cfg.Hq * (cfg.nope + cfg.rope_dim))),
        k_pe=bf16_normal(_rng("mla_rope", T, 1, salt), (T, cfg.rope_dim)),
        kv_c=bf16_normal(_rng("mla_rope", T, 2, salt), (T, cfg.kv_lora)),
        positions=_rng("mla_rope", T, 3, salt).integers(0, cfg.max_pos, T, dtype=np.int64),
        slot_mapping=_rng("mla_rope", T, 4, salt).permutation(n_slots)[:T].astype(np.int64),
    )
    if with_cache:
        r = _rng("mla_rope", 0, 5, salt).integers(
            0, 1 << 16, size=(cfg.num_blocks, cfg.block_size, cfg.kv_lora + cfg.rope_dim),
            dtype=np.uint16)
        d["kv_cache"] = (r & np.uint16(0xBFFF)).astype(np.uint16)
    return d


def mla_inputs(T: int, cfg: MlaCfg = MLA, salt: int = 0):
    """q latent [T,1536], kv latent [T,512] ~ N(0,1); weights ~ N(1, 0.1)."""
    return dict(
        q=bf16_normal(_rng("mla", T, 0, salt), (T, cfg.Hq)),
        kv=bf16_normal(_rng("mla", T, 1, salt), (T, cfg.Hkv)),
        q_w=bf16_normal(_rng("mla", 0, 2, salt), (cfg.Hq,), mean=1.0, std=0.1),
        kv_w=bf16_normal(_rng("mla", 0, 3, salt), (cfg.Hkv,), mean=1.0, std=0.1),
    )


# ---- device-resident inputs for the benchmark --------------------------------
# Same distributions as above, drawn directly on the GPU with torch's seeded
# generator (the benchmark's T = 8192 tensors are too large to draw on the host
# quickly).  Like the host generators, these only draw numbers.

def _gen(device, tag: str, T: int, salt: int = 0):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(_TAGS[tag] * 1_000_003 + int(T) * 101 + int(salt))
    return g


def _randn(g, shape, device, mean=0.0, std=1.0, dtype="bf16"):
    import torch

    a = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        a.mul_(std)
    if mean != 0.0:
        a.add_(mean)
    return a.to(torch.float16 if dtype == "f16" else torch.bfloat16)


def device_norm_inputs(T: int, H: int, device="cuda", salt: int = 0, tag: str = "norm_token",
                       dtype: str = "bf16"):
    g = _gen(device, tag, T, salt)
    return dict(x=_randn(g, (T, H), device, dtype=dtype),
                residual=_randn(g, (T, H), device, dtype=dtype),
                weight=_randn(g, (H,), device, mean=1.0, std=0.1, dtype=dtype))


def device_silu_inputs(T: int, I: int, device="cuda", salt: int = 0):
    g = _gen(device, "silu", T, salt)
    return dict(inp=_randn(g, (T, 2 * I), device, std=2.0))


def device_rope_inputs(T: int, cfg: RopeCfg = ROPE, device="cuda", salt: int = 0,
                       with_cache: bool = True):
    import torch

    g = _gen(device, "rope", T, salt)
    n_slots = cfg.num_blocks * cfg.block_size
    if T > n_slots:
        raise ValueError("more tokens than cache slots")
    d = dict(
        q=_randn(g, (T, cfg.Hq, cfg.D), device, dtype=cfg.dtype),
        k=_randn(g, (T, cfg.Hkv, cfg.D), device, dtype=cfg.dtype),
        v=_randn(g, (T, cfg.Hkv, cfg.D), device, dtype=cfg.dtype),
        positions=torch.randint(0, cfg.max_pos, (T,), generator=g, device=device,
                                dtype=torch.int64),
        slot_mapping=torch.randperm(n_slots, generator=g, device=device)[:T].contiguous(),
    )
    if with_cache:
        cache_shape = (cfg.num_blocks, cfg.block_size, cfg.Hkv, cfg.D)
        d["key_cache"] = _randn(g, cache_shape, device, dtype=cfg.dtype)
        d["value_cache"] = _randn(g, cache_shape, device, dtype=cfg.dtype)
    return d


def device_mla_inputs(T: int, cfg: MlaCfg = MLA, device="cuda", salt: int = 0):
    g = _gen(device, "mla", T, salt)
    return dict(q=_randn(g, (T, cfg.Hq), device), kv=_randn(g, (T, cfg.Hkv), device),
                q_w=_randn(g, (cfg.Hq,), device, mean=1.0, std=0.1),
                kv_w=_randn(g, (cfg.Hkv,), device, mean=1.0, std=0.1))


def device_qknorm_inputs(T: int, cfg: QkNormCfg = QKNORM, device="cuda", salt: int = 0,
                         with_cache: bool = True):
    import torch

    g = _gen(device, "qknorm", T, salt)
    n_slots = cfg.num_blocks * cfg.block_size
    d = dict(
        qkv=_randn(g, (T, (cfg.Hq + 2 * cfg.Hkv) * cfg.D), device),
        q_w=_randn(g, (cfg.D,), device, mean=1.0, std=0.1),
        k_w=_randn(g, (cfg.D,), device, mean=1.0, std=0.1),
        positions=torch.randint(0, cfg.max_pos, (T,), generator=g, device=device,
                                dtype=torch.int64),
        slot_mapping=torch.randperm(n_slots, generator=g, device=device)[:T].contiguous(),
    )
    if with_cache:
        shape = (cfg.num_blocks, cfg.block_size, cfg.Hkv, cfg.D)
        d["key_cache"] = _randn(g, shape, device)
        d["value_cache"] = _randn(g, shape, device)
    return d


def device_pad_inputs(T: int, cfg: PadCfg = PAD, device="cuda", salt: int = 0):
    return device_norm_inputs(T, cfg.H, device, salt, tag="pad", dtype=cfg.dtype)


def device_mla_rope_inputs(T: int, cfg: MlaRopeCfg = MLA_ROPE, device="cuda", salt: int = 0,
                           with_cache: bool = True):
    import torch

    g = _gen(device, "mla_rope", T, salt)
    n_slots = cfg.num_blocks * cfg.block_size
    d = dict(
        q=_randn(g, (T, cfg.Hq * (cfg.nope + cfg.rope_dim)), device),
        k_pe=_randn(g, (T, cfg.rope_dim), device),
        kv_c=_randn(g, (T, cfg.kv_lora), device),
        positions=torch.randint(0, cfg.max_pos, (T,), generator=g, device=device,
                                dtype=torch.int64),
        slot_mapping=torch.randperm(n_slots, generator=g, device=device)[:T].contiguous(),
    )
    if with_cache:
        d["kv_cache"] = _randn(g, (cfg.num_blocks, cfg.block_size, cfg.kv_lora + cfg.rope_dim),
                               device)
    return d
