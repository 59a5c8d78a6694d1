"""CPU oracle for the fused residual-add/RMSNorm/SiLU/RoPE/quant path.

TEST INFRASTRUCTURE ONLY.  This is the plain double-precision definition the
HIP library is checked against (``rra_oracle.c``).  Only ``tests/``, the smoke
check in ``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` may
import it; the library under ``rope_residual_add_amd/`` never does, and the two
share no code.

Arrays holding bf16 values are ``numpy.uint16`` bit patterns; e4m3fn codes are
``numpy.uint8``.  Each wrapper allocates and returns its outputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rra_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

Q_NONE, Q_STATIC, Q_PER_TOKEN, Q_PER_GROUP = 0, 1, 2, 3
OK, EARG, ECONTRACT = 0, -1, -2

GCC_CMD = [
    "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
    "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
    _SRC, "-o", _SO, "-lm",
]


class OracleError(RuntimeError):
    """A call the oracle rejected (bad arguments or a data-contract breach)."""

    def __init__(self, fn: str, rc: int):
        kind = {EARG: "bad arguments", ECONTRACT: "data contract violated"}.get(rc, "error")
        super().__init__(f"{fn}: {kind} (rc={rc})")
        self.rc = rc


def build() -> str:
    """Compile liboracle.so with gcc (plain C, no HIP)."""
    subprocess.check_call(GCC_CMD, cwd=_HERE)
    return _SO


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_SO)
        _declare(_lib)
    return _lib


_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int
_f32 = ctypes.c_float
_f64 = ctypes.c_double


def _declare(L: ctypes.CDLL) -> None:
    L.orc_bf16_encode.restype = ctypes.c_uint16
    L.orc_bf16_encode.argtypes = [_f64]
    L.orc_bf16_decode.restype = _f64
    L.orc_bf16_decode.argtypes = [ctypes.c_uint16]
    L.orc_e4m3fn_encode.restype = ctypes.c_uint8
    L.orc_e4m3fn_encode.argtypes = [_f64]
    L.orc_e4m3fn_encode_arith.restype = ctypes.c_uint8
    L.orc_e4m3fn_encode_arith.argtypes = [_f64]
    L.orc_e4m3fn_decode.restype = _f64
    L.orc_e4m3fn_decode.argtypes = [ctypes.c_uint8]
    L.orc_fp32_round.restype = _f32
    L.orc_fp32_round.argtypes = [_f64]
    L.orc_bf16_encode_f32_array.argtypes = [_p, _p, _i64]
    L.orc_e4m3fn_encode_f32_array.argtypes = [_p, _p, _i64]
    L.orc_e4m3fn_decode_array.argtypes = [_p, _p, _i64]
    L.orc_e4m3fn_cross_check.restype = _i64
    L.orc_e4m3fn_cross_check.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    L.orc_set_threads.argtypes = [_i32]
    L.orc_get_threads.restype = _i32
    norm = [_p, _i64, _p, _i64, _p, _f32, _i32, _i32, _f32, _p, _i64, _p, _i64, _i64]
    L.orc_fused_add_rmsnorm_quant.argtypes = norm
    L.orc_unfused_add_rmsnorm_quant.argtypes = norm
    silu = [_p, _i64, _i32, _i32, _f32, _p, _i64, _p, _i64, _i64]
    L.orc_silu_mul_quant.argtypes = silu
    L.orc_unfused_silu_mul_quant.argtypes = silu
    L.orc_f16_encode.restype = ctypes.c_uint16
    L.orc_f16_encode.argtypes = [_f64]
    L.orc_f16_decode.restype = _f64
    L.orc_f16_decode.argtypes = [ctypes.c_uint16]
    L.orc_rope_kv_write.argtypes = [
        _p, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _f64, _i64, _p, _p, _p,
        _i64, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _i32]
    L.orc_unfused_rope_kv_write.argtypes = [
        _p, _p, _i64, _p, _i64, _p, _i64, _p, _p, _i64, _f64, _i64, _p, _p, _p,
        _i64, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _i32]
    dual = [_p, _i64, _p, _f32, _p, _i64, _p, _f32, _i32, _i32, _p, _i64, _p, _p, _i64,
            _i64, _i64, _i64]
    L.orc_dual_rmsnorm_quant.argtypes = dual
    L.orc_unfused_dual_rmsnorm_quant.argtypes = dual
    qkn = [_p, _p, _i64, _p, _p, _f32, _f64, _i64, _p, _p, _p, _i32, _i64, _i32, _i32, _i32,
           _i32, _i32, _i64, _i32]
    L.orc_qk_norm_rope_kv_write.argtypes = qkn
    L.orc_unfused_qk_norm_rope_kv_write.argtypes = qkn
    L.orc_fused_add_rmsnorm_pad.argtypes = [_p, _i64, _p, _i64, _p, _f32, _p, _i64, _i64, _i64,
                                            _i64, _i32]
    L.orc_mla_rope_kv_write.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _i64, _f64, _i64, _p,
                                        _p, _i64, _i32, _i32, _i32, _i32, _i64, _i32]
    for name in ("orc_qk_norm_rope_kv_write", "orc_unfused_qk_norm_rope_kv_write",
                 "orc_fused_add_rmsnorm_pad", "orc_mla_rope_kv_write"):
        getattr(L, name).restype = _i32
    for name in ("orc_fused_add_rmsnorm_quant", "orc_unfused_add_rmsnorm_quant",
                 "orc_silu_mul_quant", "orc_unfused_silu_mul_quant", "orc_rope_kv_write",
                 "orc_unfused_rope_kv_write", "orc_dual_rmsnorm_quant",
                 "orc_unfused_dual_rmsnorm_quant"):
        getattr(L, name).restype = _i32


def _ptr(a):
    return None if a is None else a.ctypes.data


def _rows(a: np.ndarray, dtype) -> tuple[np.ndarray, int]:
    """A 2-D array with a contiguous last dimension, and its row stride in elements."""
    if a.dtype != dtype or a.ndim != 2 or a.strides[1] != a.itemsize:
        raise ValueError(f"expected a 2-D {np.dtype(dtype)} array with contiguous rows")
    return a, a.strides[0] // a.itemsize


def _check(fn: str, rc: int) -> None:
    if rc != OK:
        raise OracleError(fn, rc)


# ---- threading ------------------------------------------------------------

def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


# ---- codecs -----------------------------------------------------------------

def bf16_encode(v: float) -> int:
    return int(lib().orc_bf16_encode(float(v)))


def bf16_decode(h: int) -> float:
    return float(lib().orc_bf16_decode(int(h)))


def f16_encode(v: float) -> int:
    return int(lib().orc_f16_encode(float(v)))


def f16_decode(h: int) -> float:
    return float(lib().orc_f16_decode(int(h)))


def e4m3fn_encode(v: float) -> int:
    return int(lib().orc_e4m3fn_encode(float(v)))


def e4m3fn_encode_arith(v: float) -> int:
    return int(lib().orc_e4m3fn_encode_arith(float(v)))


def e4m3fn_decode(c: int) -> float:
    return float(lib().orc_e4m3fn_decode(int(c)))


def fp32_round(v: float) -> float:
    return float(lib().orc_fp32_round(float(v)))


def bf16_encode_f32(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().orc_bf16_encode_f32_array(_ptr(a), _ptr(out), a.size)
    return out


def e4m3fn_encode_f32(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint8)
    lib().orc_e4m3fn_encode_f32_array(_ptr(a), _ptr(out), a.size)
    return out


def e4m3fn_decode_array(c: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().orc_e4m3fn_decode_array(_ptr(c), _ptr(out), c.size)
    return out


def bf16_to_f64(h: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (exact in float64)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3fn_cross_check(begin: int, end: int) -> int:
    return int(lib().orc_e4m3fn_cross_check(begin, end))


# ---- fused ops and their unfused compositions --------------------------------

DT_BF16, DT_F16 = 0, 1


def _dtype(name: str) -> int:
    codes = {"bf16": DT_BF16, "f16": DT_F16}
    if name not in codes:
        raise ValueError(f"element type must be 'bf16' or 'f16', not {name!r}")
    return codes[name]


def _scales_shape(mode: int, T: int, H: int, g: int):
    if mode == Q_PER_TOKEN:
        return (T,)
    if mode == Q_PER_GROUP:
        return (T, H // g if g > 0 and H % g == 0 else 0)
    return None


def _norm(fn: str, x, residual, weight, eps, quant_mode, group_size, static_scale):
    x, xs = _rows(x, np.uint16)
    T, H = x.shape
    res = None
    rs = 0
    if residual is not None:
        res, rs = _rows(residual.copy(), np.uint16)
    w = np.ascontiguousarray(weight, dtype=np.uint16)
    out = np.zeros((T, H), np.uint8)
    ss = _scales_shape(quant_mode, T, H, group_size)
    scales = np.zeros(ss, np.float32) if ss is not None else None
    rc = getattr(lib(), fn)(_ptr(x), xs, _ptr(res), rs, _ptr(w), eps, quant_mode,
                            group_size, static_scale, _ptr(out), H, _ptr(scales), T, H)
    _check(fn, rc)
    return out, scales, res


def fused_add_rmsnorm_quant(x, residual, weight, eps, quant_mode, group_size=0,
                            static_scale=0.0):
    """Returns (codes [T,H] u8, scales or None, updated residual or None)."""
    return _norm("orc_fused_add_rmsnorm_quant", x, residual, weight, eps, quant_mode,
                 group_size, static_scale)


def unfused_add_rmsnorm_quant(x, residual, weight, eps, quant_mode, group_size=0,
                              static_scale=0.0):
    return _norm("orc_unfused_add_rmsnorm_quant", x, residual, weight, eps, quant_mode,
                 group_size, static_scale)


def _silu(fn: str, inp, quant_mode, group_size, static_scale):
    inp, s = _rows(inp, np.uint16)
    T, two_i = inp.shape
    I = two_i // 2
    out = np.zeros((T, I), np.uint8)
    ss = _scales_shape(quant_mode, T, I, group_size)
    scales = np.zeros(ss, np.float32) if ss is not None else None
    rc = getattr(lib(), fn)(_ptr(inp), s, quant_mode, group_size, static_scale, _ptr(out), I,
                            _ptr(scales), T, I)
    _check(fn, rc)
    return out, scales


def silu_mul_quant(inp, quant_mode, group_size=0, static_scale=0.0):
    """inp: [T, 2I] bf16 bits (gate | up).  Returns (codes [T,I], scales or None)."""
    return _silu("orc_silu_mul_quant", inp, quant_mode, group_size, static_scale)


def unfused_silu_mul_quant(inp, quant_mode, group_size=0, static_scale=0.0):
    return _silu("orc_unfused_silu_mul_quant", inp, quant_mode, group_size, static_scale)


def _head_rows(a, H, D):
    """[T, H, D] (or [T, H*D]) bf16 bits with contiguous heads -> (array, token stride)."""
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise ValueError("expected uint16 (bf16 bits)")
    if a.ndim == 3:
        if a.shape[1:] != (H, D) or a.strides[2] != 2 or a.strides[1] != 2 * D:
            raise ValueError("heads must be contiguous [H, D]")
        return a, a.strides[0] // 2
    return _rows(a, np.uint16)


def rope_kv_write(positions, q, k, v, theta, max_pos, slot_mapping, key_cache, value_cache,
                  Hq, Hkv, D, rot_dim=None, is_neox=True, dtype="bf16"):
    """Returns (q_out, key_cache', value_cache'); the input caches are not modified.
    q, k, v and the caches are uint16 bit patterns of dtype ("bf16" or "f16")."""
    rot_dim = D if rot_dim is None else rot_dim
    positions = np.ascontiguousarray(positions, dtype=np.int64)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    T = positions.shape[0]
    q, qs = _head_rows(q, Hq, D)
    k, ks = _head_rows(k, Hkv, D)
    v, vs = _head_rows(v, Hkv, D)
    q_out = np.zeros((T, Hq, D), np.uint16)
    kc = np.ascontiguousarray(key_cache, dtype=np.uint16).copy()
    vc = np.ascontiguousarray(value_cache, dtype=np.uint16).copy()
    num_blocks, block_size = kc.shape[0], kc.shape[1]
    rc = lib().orc_rope_kv_write(_ptr(positions), _ptr(q), qs, _ptr(q_out), Hq * D, _ptr(k), ks,
                                 _ptr(v), vs, float(theta), int(max_pos), _ptr(slots), _ptr(kc),
                                 _ptr(vc), T, Hq, Hkv, D, rot_dim, block_size, num_blocks,
                                 int(bool(is_neox)), _dtype(dtype))
    _check("orc_rope_kv_write", rc)
    return q_out, kc, vc


def unfused_rope_kv_write(positions, q, k, v, theta, max_pos, slot_mapping, key_cache,
                          value_cache, Hq, Hkv, D, rot_dim=None, is_neox=True, dtype="bf16"):
    """Returns (q_out, k_out, key_cache', value_cache')."""
    rot_dim = D if rot_dim is None else rot_dim
    positions = np.ascontiguousarray(positions, dtype=np.int64)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    T = positions.shape[0]
    q, qs = _head_rows(q, Hq, D)
    k, ks = _head_rows(k, Hkv, D)
    v, vs = _head_rows(v, Hkv, D)
    q_out = np.zeros((T, Hq, D), np.uint16)
    k_out = np.zeros((T, Hkv, D), np.uint16)
    kc = np.ascontiguousarray(key_cache, dtype=np.uint16).copy()
    vc = np.ascontiguousarray(value_cache, dtype=np.uint16).copy()
    num_blocks, block_size = kc.shape[0], kc.shape[1]
    rc = lib().orc_unfused_rope_kv_write(
        _ptr(positions), _ptr(q), qs, _ptr(q_out), Hq * D, _ptr(k), ks, _ptr(k_out), _ptr(v),
        vs, float(theta), int(max_pos), _ptr(slots), _ptr(kc), _ptr(vc), T, Hq, Hkv, D,
        rot_dim, block_size, num_blocks, int(bool(is_neox)), _dtype(dtype))
    _check("orc_unfused_rope_kv_write", rc)
    return q_out, k_out, kc, vc


def _dual(fn, q, q_w, eps_q, kv, kv_w, eps_kv, q_quant_mode, group_size):
    q, qs = _rows(q, np.uint16)
    kv, kvs = _rows(kv, np.uint16)
    T, Hq = q.shape
    Hkv = kv.shape[1]
    if q_quant_mode == Q_NONE:
        q_out = np.zeros((T, Hq), np.uint16)
    else:
        q_out = np.zeros((T, Hq), np.uint8)
    ss = _scales_shape(q_quant_mode, T, Hq, group_size)
    q_scales = np.zeros(ss, np.float32) if ss is not None else None
    kv_out = np.zeros((T, Hkv), np.uint16)
    rc = getattr(lib(), fn)(_ptr(q), qs, _ptr(np.ascontiguousarray(q_w, np.uint16)), eps_q,
                            _ptr(kv), kvs, _ptr(np.ascontiguousarray(kv_w, np.uint16)), eps_kv,
                            q_quant_mode, group_size, _ptr(q_out), Hq, _ptr(q_scales),
                            _ptr(kv_out), Hkv, T, Hq, Hkv)
    _check(fn, rc)
    return q_out, q_scales, kv_out


def dual_rmsnorm_quant(q, q_w, eps_q, kv, kv_w, eps_kv, q_quant_mode, group_size=0):
    """Returns (q_out [bf16 bits or e4m3fn codes], q_scales or None, kv_out bf16 bits)."""
    return _dual("orc_dual_rmsnorm_quant", q, q_w, eps_q, kv, kv_w, eps_kv, q_quant_mode,
                 group_size)


def unfused_dual_rmsnorm_quant(q, q_w, eps_q, kv, kv_w, eps_kv, q_quant_mode, group_size=0):
    return _dual("orc_unfused_dual_rmsnorm_quant", q, q_w, eps_q, kv, kv_w, eps_kv,
                 q_quant_mode, group_size)


# ---- next rows ----------------------------------------------------------------

def _qkn(fn, positions, qkv, q_weight, k_weight, eps, theta, max_pos, Hq, Hkv, D,
         slot_mapping=None, key_cache=None, value_cache=None, write_k=False, rot_dim=None,
         is_neox=True):
    rot_dim = D if rot_dim is None else rot_dim
    positions = np.ascontiguousarray(positions, dtype=np.int64)
    T = positions.shape[0]
    qkv = np.array(qkv, dtype=np.uint16, copy=True).reshape(T, -1)
    qkv, qs = _rows(qkv, np.uint16)
    slots = None if slot_mapping is None else np.ascontiguousarray(slot_mapping, dtype=np.int64)
    kc = vc = None
    num_blocks, block_size = 1, 1
    if key_cache is not None:
        kc = np.ascontiguousarray(key_cache, dtype=np.uint16).copy()
        vc = np.ascontiguousarray(value_cache, dtype=np.uint16).copy()
        num_blocks, block_size = kc.shape[0], kc.shape[1]
    rc = getattr(lib(), fn)(_ptr(positions), _ptr(qkv), qs,
                            _ptr(np.ascontiguousarray(q_weight, np.uint16)),
                            _ptr(np.ascontiguousarray(k_weight, np.uint16)), float(eps),
                            float(theta), int(max_pos), _ptr(slots), _ptr(kc), _ptr(vc),
                            int(bool(write_k)), T, Hq, Hkv, D, rot_dim, block_size, num_blocks,
                            int(bool(is_neox)))
    _check(fn, rc)
    return qkv, kc, vc


def qk_norm_rope_kv_write(positions, qkv, q_weight, k_weight, eps, theta, max_pos, Hq, Hkv, D,
                          **kw):
    """Per-head RMSNorm of q and k in the packed qkv rows, then RoPE; optional
    paged cache write.  Returns (qkv', key_cache' or None, value_cache' or None);
    the inputs are not modified."""
    return _qkn("orc_qk_norm_rope_kv_write", positions, qkv, q_weight, k_weight, eps, theta,
                max_pos, Hq, Hkv, D, **kw)


def unfused_qk_norm_rope_kv_write(positions, qkv, q_weight, k_weight, eps, theta, max_pos, Hq,
                                  Hkv, D, **kw):
    return _qkn("orc_unfused_qk_norm_rope_kv_write", positions, qkv, q_weight, k_weight, eps,
                theta, max_pos, Hq, Hkv, D, **kw)


def fused_add_rmsnorm_pad(x, residual, weight, eps, H_pad, dtype="bf16"):
    """Returns (out [T, H_pad] bit patterns of dtype ("bf16" or "f16"), updated
    residual or None)."""
    x, xs = _rows(x, np.uint16)
    T, H = x.shape
    res, rs = (None, 0)
    if residual is not None:
        res, rs = _rows(residual.copy(), np.uint16)
    out = np.full((T, H_pad), 0xFFFF, np.uint16)  # every column must be written
    rc = lib().orc_fused_add_rmsnorm_pad(_ptr(x), xs, _ptr(res), rs,
                                         _ptr(np.ascontiguousarray(weight, np.uint16)),
                                         float(eps), _ptr(out), H_pad, T, H, H_pad,
                                         _dtype(dtype))
    _check("orc_fused_add_rmsnorm_pad", rc)
    return out, res


def mla_rope_kv_write(positions, q, k_pe, kv_c, theta, max_pos, slot_mapping, kv_cache, Hq,
                      rope_dim, q_head_stride=None, q_pe_offset=0, is_neox=False):
    """q: [T, Hq * q_head_stride] bf16 rows whose heads hold their rope part at
    columns [q_pe_offset, q_pe_offset + rope_dim); k_pe: [T, rope_dim];
    kv_c: [T, kv_lora]; kv_cache: [num_blocks, block_size, kv_lora + rope_dim].
    Returns (q', kv_cache'); the inputs are not modified."""
    positions = np.ascontiguousarray(positions, dtype=np.int64)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    T = positions.shape[0]
    q = np.array(q, dtype=np.uint16, copy=True).reshape(T, -1)
    q, qs = _rows(q, np.uint16)
    q_head_stride = rope_dim if q_head_stride is None else q_head_stride
    k_pe, ks = _rows(np.ascontiguousarray(k_pe, np.uint16).reshape(T, -1), np.uint16)
    kv_c, cs = _rows(np.ascontiguousarray(kv_c, np.uint16).reshape(T, -1), np.uint16)
    cache = np.ascontiguousarray(kv_cache, dtype=np.uint16).copy()
    num_blocks, block_size, width = cache.shape
    kv_lora = kv_c.shape[1]
    if width != kv_lora + rope_dim:
        raise ValueError("cache width must be kv_lora + rope_dim")
    q_view = q[:, q_pe_offset:]
    rc = lib().orc_mla_rope_kv_write(_ptr(positions), q_view.ctypes.data, qs, q_head_stride,
                                     _ptr(k_pe), ks, _ptr(kv_c), cs, float(theta),
                                     int(max_pos), _ptr(slots), _ptr(cache), T, Hq, kv_lora,
                                     rope_dim, block_size, num_blocks, int(bool(is_neox)))
    _check("orc_mla_rope_kv_write", rc)
    return q, cache
