"""Fused residual-add / RMSNorm / SiLU / RoPE / FP8-quant kernels for AMD MI355X.

Python binding of ``librra.so`` (hand-written HIP for gfx950).  Every function
here only marshals torch tensors into the C ABI declared in ``include/rra.h``
and raises ``RRAError`` on a non-zero status; all computation happens in the
library's kernels, on the tensors' device and the current torch stream.  PyTorch
is used only for device memory and streams.

The library must be built first (``python -m rope_residual_add_amd.build`` or
``__graft_entry__.build()``); importing this package without it fails loudly.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch  # imported first so that librra.so binds to torch's HIP runtime

from .build import SO as LIBRARY_PATH

Q_NONE, Q_STATIC, Q_PER_TOKEN, Q_PER_GROUP = 0, 1, 2, 3
_QUANT_NAMES = {"none": Q_NONE, "static": Q_STATIC, "per_token": Q_PER_TOKEN,
                "per_group": Q_PER_GROUP}

EXPORTS = ("rra_abi_version", "rra_status_string", "fused_add_rmsnorm_quant", "silu_mul_quant",
           "rope_cos_sin_cache", "rope_kv_write", "dual_rmsnorm_quant", "qk_norm_rope_kv_write",
           "fused_add_rmsnorm_pad", "mla_rope_kv_write", "rra_e4m3fn_encode", "rra_stream_copy")


class RRAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


ABI_VERSION = 6  # RRA_ABI_VERSION of include/rra.h
BF16, F16 = 0, 1  # enum rra_dtype
_ELEM = {torch.bfloat16: BF16, torch.float16: F16}

_lib = None
_p, _i64, _i32, _f32, _f64 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                              ctypes.c_double)


def lib() -> ctypes.CDLL:
    """The loaded librra.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY_PATH):
            raise ImportError(f"{LIBRARY_PATH} is missing: build it with "
                              "`python -m rope_residual_add_amd.build`")
        L = ctypes.CDLL(LIBRARY_PATH)
        L.rra_abi_version.restype = _i32
        if L.rra_abi_version() != ABI_VERSION:
            raise ImportError(f"{LIBRARY_PATH} has ABI {L.rra_abi_version()}, this binding "
                              f"needs {ABI_VERSION}: rebuild it")
        L.rra_status_string.restype = ctypes.c_char_p
        L.rra_status_string.argtypes = [_i32]
        L.fused_add_rmsnorm_quant.argtypes = [_p, _i64, _p, _i64, _p, _f32, _i32, _i32, _p, _p,
                                              _i64, _p, _i64, _i64, _p]
        L.silu_mul_quant.argtypes = [_p, _i64, _i32, _i32, _p, _p, _i64, _p, _i64, _i64, _p]
        L.rope_cos_sin_cache.argtypes = [_p, _i64, _i32, _f64, _p]
        L.rope_kv_write.argtypes = [_p, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _p,
                                    _p, _i64, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _p]
        L.dual_rmsnorm_quant.argtypes = [_p, _i64, _p, _f32, _p, _i64, _p, _f32, _i32, _i32, _p,
                                         _i64, _p, _p, _i64, _i64, _i64, _i64, _p]
        L.qk_norm_rope_kv_write.argtypes = [_p, _p, _i64, _p, _p, _f32, _p, _i64, _p, _p, _p,
                                            _i32, _i64, _i32, _i32, _i32, _i32, _i32, _i64,
                                            _i32, _p]
        L.fused_add_rmsnorm_pad.argtypes = [_p, _i64, _p, _i64, _p, _f32, _p, _i64, _i64, _i64,
                                            _i64, _i32, _p]
        L.mla_rope_kv_write.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _p,
                                        _i64, _i32, _i32, _i32, _i32, _i64, _i32, _p]
        L.rra_e4m3fn_encode.argtypes = [_p, _p, _i64, _p]
        L.rra_stream_copy.argtypes = [_p, _p, _i64, _i32, _p]
        for name in EXPORTS[2:]:
            getattr(L, name).restype = _i32
        _lib = L
    return _lib


def abi_version() -> int:
    return int(lib().rra_abi_version())


def status_string(status: int) -> str:
    return lib().rra_status_string(int(status)).decode()


# ---- marshalling helpers -----------------------------------------------------

def _mode(m) -> int:
    return _QUANT_NAMES[m] if isinstance(m, str) else int(m)


def _ptr(t):
    return None if t is None else t.data_ptr()


# The current stream and device are read straight from torch's C++ side where it
# offers them: torch.cuda.current_stream() builds a Stream object (~3 us a call)
# and entering torch.cuda.device costs ~1.4 us, against ~3.5 us for the whole
# C call with its kernel launch.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_current_device = getattr(torch._C, "_cuda_getDevice", None)
_SAME_DEVICE = contextlib.nullcontext()


def _stream(t: torch.Tensor):
    """The current torch stream of t's device, as the hipStream_t the C ABI takes."""
    if _raw_stream is not None:
        return _raw_stream(t.device.index)
    return torch.cuda.current_stream(t.device).cuda_stream


def _on_device(dev: torch.device):
    """Makes dev the current device for a call (the library launches on the
    current device); a no-op context when it already is."""
    if _current_device is not None and _current_device() == dev.index:
        return _SAME_DEVICE
    return torch.cuda.device(dev)


# Every tensor an entry point touches is checked here before the call: device,
# dtype, shape (rows included) and layout.  The kernels trust the sizes they
# are given, so a tensor smaller than its stated shape would be read or
# written out of bounds.

def _need_cuda(name: str, t: torch.Tensor, dtypes, device=None) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other operands on {device}")


def _vector(name: str, t: torch.Tensor, n: int, dtypes=(torch.bfloat16,), device=None) -> None:
    _need_cuda(name, t, dtypes, device)
    if t.dim() != 1 or t.shape[0] != n or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [{n}] tensor")


def _rows(name: str, t: torch.Tensor, dtypes, width: int | None = None, rows: int | None = None,
          device=None) -> int:
    """Check a [rows, width] tensor with contiguous rows; return its row stride."""
    _need_cuda(name, t, dtypes, device)
    if t.dim() != 2 or (t.numel() > 0 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with contiguous rows")
    if width is not None and t.shape[1] != width:
        raise ValueError(f"{name} must have {width} columns, got {t.shape[1]}")
    if rows is not None and t.shape[0] != rows:
        raise ValueError(f"{name} must have {rows} rows, got {t.shape[0]}")
    return t.stride(0)


def _heads(name: str, t: torch.Tensor, H: int, D: int, dtypes=(torch.bfloat16,),
           rows: int | None = None, device=None) -> int:
    """Check a [T, H, D] (or [T, H*D]) tensor whose heads are contiguous."""
    _need_cuda(name, t, dtypes, device)
    if t.dim() == 3:
        if tuple(t.shape[1:]) != (H, D) or (t.numel() > 0 and (t.stride(2) != 1 or t.stride(1) != D)):
            raise ValueError(f"{name} must be [T, {H}, {D}] with contiguous heads")
        if rows is not None and t.shape[0] != rows:
            raise ValueError(f"{name} must have {rows} tokens, got {t.shape[0]}")
        return t.stride(0)
    return _rows(name, t, dtypes, H * D, rows, device)


def _tokens(name: str, t: torch.Tensor, T: int, device) -> None:
    """A contiguous [T] int64 tensor (positions, slot mapping)."""
    _vector(name, t, T, (torch.int64,), device)


def _exact(name: str, t: torch.Tensor, shape, dtypes, device) -> None:
    """A contiguous tensor of exactly this shape (scales, tables, codes)."""
    _need_cuda(name, t, dtypes, device)
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {list(shape)} tensor, got "
                         f"{list(t.shape)}")


def _static(t, device) -> None:
    """The static scale: a device fp32 tensor holding at least one value."""
    _need_cuda("static_scale", t, (torch.float32,), device)
    if t.numel() < 1:
        raise ValueError("static_scale must hold one value")


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise RRAError(fn, status)


_BF16 = (torch.bfloat16,)
_FP8 = (torch.float8_e4m3fn, torch.uint8)


def _scales_shape(mode: int, T: int, H: int, g: int):
    if mode == Q_PER_TOKEN:
        return (T,)
    if mode == Q_PER_GROUP:
        return (T, H // g)
    return None


# ---- the fused ops -------------------------------------------------------------

def fused_add_rmsnorm_quant(x, residual, weight, eps, quant_mode, group_size=0,
                            static_scale=None, out=None, scales=None):
    """Residual add + RMSNorm + FP8 quant (residual updated in place).

    x, residual: [T, H] bf16 (residual may be None); weight: [H] bf16;
    static_scale: [1] fp32 device tensor (static mode).  Returns (out, scales):
    out [T, H] float8_e4m3fn, scales [T] / [T, H/g] fp32 or None."""
    mode = _mode(quant_mode)
    xs = _rows("x", x, _BF16)
    T, H = x.shape
    dev = x.device
    rs = _rows("residual", residual, _BF16, H, T, dev) if residual is not None else 0
    _vector("weight", weight, H, device=dev)
    if static_scale is not None:
        _static(static_scale, dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.float8_e4m3fn, device=dev)
    os_ = _rows("out", out, _FP8, H, T, dev)
    shape = _scales_shape(mode, T, H, group_size or 1)
    if scales is None and shape is not None:
        scales = torch.empty(shape, dtype=torch.float32, device=dev)
    if scales is not None and shape is not None:
        _exact("scales", scales, shape, (torch.float32,), dev)
    with _on_device(x.device):
        st = lib().fused_add_rmsnorm_quant(
            _ptr(x), xs, _ptr(residual), rs, _ptr(weight), float(eps), mode,
            int(group_size), _ptr(static_scale), _ptr(out), os_, _ptr(scales), T, H, _stream(x))
    _check("fused_add_rmsnorm_quant", st)
    return out, scales


def silu_mul_quant(inp, quant_mode, group_size=0, static_scale=None, out=None, scales=None):
    """SiLU-and-Mul + FP8 quant.  inp: [T, 2I] bf16 (gate | up).
    Returns (out [T, I] float8_e4m3fn, scales [T, I/g] fp32 or None)."""
    mode = _mode(quant_mode)
    s = _rows("inp", inp, _BF16)
    T, two_i = inp.shape
    if two_i % 2:
        raise ValueError("inp must hold gate and up halves of equal width")
    I = two_i // 2
    dev = inp.device
    if static_scale is not None:
        _static(static_scale, dev)
    if out is None:
        out = torch.empty((T, I), dtype=torch.float8_e4m3fn, device=dev)
    os_ = _rows("out", out, _FP8, I, T, dev)
    shape = _scales_shape(mode, T, I, group_size or 1)
    if scales is None and shape is not None:
        scales = torch.empty(shape, dtype=torch.float32, device=dev)
    if scales is not None and shape is not None:
        _exact("scales", scales, shape, (torch.float32,), dev)
    with _on_device(inp.device):
        st = lib().silu_mul_quant(_ptr(inp), s, mode, int(group_size), _ptr(static_scale),
                                  _ptr(out), os_, _ptr(scales), T, I, _stream(inp))
    _check("silu_mul_quant", st)
    return out, scales


def rope_cos_sin_cache(max_pos: int, rot_dim: int, theta: float, device="cuda", out=None):
    """[max_pos, rot_dim] fp32 table: cos of the rot_dim/2 angles, then sin."""
    if out is None:
        out = torch.empty((max_pos, rot_dim), dtype=torch.float32, device=device)
    _exact("out", out, (max_pos, rot_dim), (torch.float32,), out.device)
    with _on_device(out.device):
        st = lib().rope_cos_sin_cache(_ptr(out), int(max_pos), int(rot_dim), float(theta),
                                      _stream(out))
    _check("rope_cos_sin_cache", st)
    return out


def rope_kv_write(positions, q, k, v, cos_sin, slot_mapping, key_cache, value_cache,
                  q_out=None, is_neox=True):
    """RoPE of q and k + paged KV-cache write of rotated k and v.

    q: [T, Hq, D], k, v: [T, Hkv, D] bf16 or fp16 (one type for q, k, v,
    q_out and both caches); cos_sin: [max_pos, rot_dim] fp32;
    positions, slot_mapping: [T] int64 (slot < 0 = padding);
    caches: [num_blocks, block_size, Hkv, D].  q_out defaults to q
    (in place).  is_neox selects GPT-NeoX pairs (i, i + D/2), else GPT-J
    pairs (2i, 2i + 1).  Returns q_out."""
    _need_cuda("q", q, tuple(_ELEM))
    dev, elem = q.device, (q.dtype,)
    _need_cuda("key_cache", key_cache, elem, dev)
    if key_cache.dim() != 4:
        raise ValueError("key_cache must be [num_blocks, block_size, Hkv, D]")
    num_blocks, block_size, Hkv, D = key_cache.shape
    for name, c in (("key_cache", key_cache), ("value_cache", value_cache)):
        _exact(name, c, (num_blocks, block_size, Hkv, D), elem, dev)
    if q.dim() not in (2, 3) or D == 0:
        raise ValueError("q must be [T, Hq, D] or [T, Hq * D]")
    T = q.shape[0]
    Hq = q.shape[1] if q.dim() == 3 else q.shape[1] // D
    _tokens("positions", positions, T, dev)
    _tokens("slot_mapping", slot_mapping, T, dev)
    if cos_sin.dim() != 2:
        raise ValueError("cos_sin must be [max_pos, rot_dim]")
    _exact("cos_sin", cos_sin, cos_sin.shape, (torch.float32,), dev)
    if q_out is None:
        q_out = q
    qs = _heads("q", q, Hq, D, elem, T, dev)
    qos = _heads("q_out", q_out, Hq, D, elem, T, dev)
    ks, vs = _heads("k", k, Hkv, D, elem, T, dev), _heads("v", v, Hkv, D, elem, T, dev)
    max_pos, rot_dim = cos_sin.shape
    with _on_device(q.device):
        st = lib().rope_kv_write(
            _ptr(positions), _ptr(q), qs, _ptr(q_out), qos, _ptr(k), ks, _ptr(v), vs,
            _ptr(cos_sin), max_pos, _ptr(slot_mapping), _ptr(key_cache), _ptr(value_cache), T,
            Hq, Hkv, D, rot_dim, block_size, num_blocks, int(bool(is_neox)), _ELEM[q.dtype],
            _stream(q))
    _check("rope_kv_write", st)
    return q_out


def dual_rmsnorm_quant(q, q_weight, eps_q, kv, kv_weight, eps_kv, q_quant_mode="none",
                       group_size=0, q_out=None, q_scales=None, kv_out=None):
    """MLA dual RMSNorm of the q and kv latents in one launch; the q side is
    optionally FP8-quantized.  Returns (q_out, q_scales or None, kv_out)."""
    mode = _mode(q_quant_mode)
    qs = _rows("q", q, _BF16)
    T, Hq = q.shape
    dev = q.device
    kvs = _rows("kv", kv, _BF16, rows=T, device=dev)
    Hkv = kv.shape[1]
    _vector("q_weight", q_weight, Hq, device=dev)
    _vector("kv_weight", kv_weight, Hkv, device=dev)
    if q_out is None:
        dt = torch.bfloat16 if mode == Q_NONE else torch.float8_e4m3fn
        q_out = torch.empty((T, Hq), dtype=dt, device=dev)
    qos = _rows("q_out", q_out, _BF16 if mode == Q_NONE else _FP8, Hq, T, dev)
    shape = _scales_shape(mode, T, Hq, group_size or 1)
    if q_scales is None and shape is not None:
        q_scales = torch.empty(shape, dtype=torch.float32, device=dev)
    if q_scales is not None and shape is not None:
        _exact("q_scales", q_scales, shape, (torch.float32,), dev)
    if kv_out is None:
        kv_out = torch.empty((T, Hkv), dtype=torch.bfloat16, device=dev)
    kvos = _rows("kv_out", kv_out, _BF16, Hkv, T, dev)
    with _on_device(q.device):
        st = lib().dual_rmsnorm_quant(
            _ptr(q), qs, _ptr(q_weight), float(eps_q), _ptr(kv), kvs,
            _ptr(kv_weight), float(eps_kv), mode, int(group_size), _ptr(q_out), qos,
            _ptr(q_scales), _ptr(kv_out), kvos, T, Hq, Hkv, _stream(q))
    _check("dual_rmsnorm_quant", st)
    return q_out, q_scales, kv_out


def qk_norm_rope_kv_write(positions, qkv, q_weight, k_weight, eps, cos_sin, Hq, Hkv, D,
                          slot_mapping=None, key_cache=None, value_cache=None, write_k=None,
                          is_neox=True):
    """Per-head RMSNorm of q and k inside the packed qkv rows, then RoPE; q is
    updated in place in qkv (and k with write_k).  With slot_mapping, rotated
    k and v go to the paged caches [num_blocks, block_size, Hkv, D].
    write_k defaults to True without a cache (k's only destination is then
    qkv; False is refused there) and to False with one.
    qkv: [T, (Hq + 2 Hkv) D] bf16 with contiguous rows.  Returns qkv."""
    if write_k is None:
        write_k = slot_mapping is None
    qs = _rows("qkv", qkv, _BF16, (Hq + 2 * Hkv) * D)
    T, dev = qkv.shape[0], qkv.device
    _tokens("positions", positions, T, dev)
    if cos_sin.dim() != 2:
        raise ValueError("cos_sin must be [max_pos, rot_dim]")
    _exact("cos_sin", cos_sin, cos_sin.shape, (torch.float32,), dev)
    _vector("q_weight", q_weight, D, device=dev)
    _vector("k_weight", k_weight, D, device=dev)
    num_blocks = block_size = 0
    if slot_mapping is not None:
        _tokens("slot_mapping", slot_mapping, T, dev)
        _need_cuda("key_cache", key_cache, _BF16, dev)
        if key_cache.dim() != 4 or tuple(key_cache.shape[2:]) != (Hkv, D):
            raise ValueError("key_cache must be a contiguous [num_blocks, block_size, Hkv, D] "
                             "tensor")
        num_blocks, block_size = key_cache.shape[:2]
        for name, c in (("key_cache", key_cache), ("value_cache", value_cache)):
            _exact(name, c, (num_blocks, block_size, Hkv, D), _BF16, dev)
    max_pos, rot_dim = cos_sin.shape
    with _on_device(qkv.device):
        st = lib().qk_norm_rope_kv_write(
            _ptr(positions), _ptr(qkv), qs, _ptr(q_weight), _ptr(k_weight), float(eps),
            _ptr(cos_sin), max_pos, _ptr(slot_mapping), _ptr(key_cache), _ptr(value_cache),
            int(bool(write_k)), T, Hq, Hkv, D, rot_dim, block_size, num_blocks,
            int(bool(is_neox)), _stream(qkv))
    _check("qk_norm_rope_kv_write", st)
    return qkv


def fused_add_rmsnorm_pad(x, residual, weight, eps, H_pad, out=None):
    """Residual add + RMSNorm, written into out[:, :H] with out[:, H:H_pad] = 0
    (residual updated in place).  x, residual, weight and out share one element
    type, bf16 or fp16.  Returns out [T, H_pad]."""
    _need_cuda("x", x, tuple(_ELEM))
    elem, dev = (x.dtype,), x.device
    xs = _rows("x", x, elem)
    T, H = x.shape
    rs = _rows("residual", residual, elem, H, T, dev) if residual is not None else 0
    _vector("weight", weight, H, elem, dev)
    if out is None:
        out = torch.empty((T, H_pad), dtype=x.dtype, device=dev)
    os_ = _rows("out", out, elem, H_pad, T, dev)
    with _on_device(x.device):
        st = lib().fused_add_rmsnorm_pad(_ptr(x), xs, _ptr(residual), rs, _ptr(weight),
                                         float(eps), _ptr(out), os_, T, H, H_pad,
                                         _ELEM[x.dtype], _stream(x))
    _check("fused_add_rmsnorm_pad", st)
    return out


def mla_rope_kv_write(positions, q, k_pe, kv_c, cos_sin, slot_mapping, kv_cache, Hq, rope_dim,
                      q_head_stride, q_pe_offset, is_neox=False):
    """RoPE of the rope part of each q head (in place in q: head h of a row
    starts at h * q_head_stride, its rope part at q_pe_offset) and of k_pe, and
    the MLA cache write of [kv_c | rotated k_pe] at each token's slot.
    q: [T, Hq * q_head_stride] bf16; k_pe: [T, rope_dim]; kv_c: [T, kv_lora];
    kv_cache: [num_blocks, block_size, kv_lora + rope_dim].  Returns q."""
    qs = _rows("q", q, _BF16)
    T, dev = q.shape[0], q.device
    ks = _rows("k_pe", k_pe, _BF16, rope_dim, T, dev)
    cs = _rows("kv_c", kv_c, _BF16, rows=T, device=dev)
    kv_lora = kv_c.shape[1]
    _tokens("positions", positions, T, dev)
    _tokens("slot_mapping", slot_mapping, T, dev)
    if cos_sin.dim() != 2 or cos_sin.shape[1] != rope_dim:
        raise ValueError(f"cos_sin must be [max_pos, {rope_dim}]")
    _exact("cos_sin", cos_sin, cos_sin.shape, (torch.float32,), dev)
    _need_cuda("kv_cache", kv_cache, _BF16, dev)
    if kv_cache.dim() != 3 or kv_cache.shape[2] != kv_lora + rope_dim or \
            not kv_cache.is_contiguous():
        raise ValueError("kv_cache must be a contiguous [num_blocks, block_size, "
                         "kv_lora + rope_dim] tensor")
    if q.shape[1] < (Hq - 1) * q_head_stride + q_pe_offset + rope_dim:
        raise ValueError("q is too narrow for Hq heads of q_head_stride")
    num_blocks, block_size = kv_cache.shape[:2]
    max_pos = cos_sin.shape[0]
    with _on_device(q.device):
        st = lib().mla_rope_kv_write(
            _ptr(positions), q.data_ptr() + 2 * q_pe_offset if q.numel() else None, qs,
            q_head_stride, _ptr(k_pe), ks, _ptr(kv_c), cs, _ptr(cos_sin), max_pos,
            _ptr(slot_mapping), _ptr(kv_cache), T, Hq, kv_lora, rope_dim, block_size,
            num_blocks, int(bool(is_neox)), _stream(q))
    _check("mla_rope_kv_write", st)
    return q


def e4m3fn_encode(x, out=None):
    """fp32 -> e4m3fn codes with the kernels' device conversion (diagnostic)."""
    _need_cuda("x", x, (torch.float32,))
    x = x.contiguous()
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _exact("out", out, x.shape, (torch.uint8,), x.device)
    with _on_device(x.device):
        st = lib().rra_e4m3fn_encode(_ptr(x), _ptr(out), x.numel(), _stream(x))
    _check("rra_e4m3fn_encode", st)
    return out


def stream_copy(src, dst, vectors_per_lane=1):
    """dst <- src (same byte size, contiguous, non-overlapping) with the fused
    kernels' streaming loads and stores, vectors_per_lane (1, 2, 4 or 8)
    16-byte vectors per lane: the bandwidth yardstick (diagnostic)."""
    for name, t in (("src", src), ("dst", dst)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a GPU tensor")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("stream_copy: src and dst differ in size")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("stream_copy: src and dst must be contiguous")
    with _on_device(src.device):
        st = lib().rra_stream_copy(_ptr(src), _ptr(dst), nbytes, int(vectors_per_lane),
                                   _stream(src))
    _check("rra_stream_copy", st)
    return dst
