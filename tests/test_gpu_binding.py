"""The Python binding checks every tensor before it calls the library: rows,
widths, dtypes, devices and the scale buffers a caller passes in.  The
kernels trust the sizes they are given, so each mismatch below would
otherwise read or write outside a tensor.  Every call here is refused on the
host; nothing is launched."""
import pytest

from gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rra():
    require_gpu()
    import rope_residual_add_amd as r

    r.lib()
    return r


def _t(*shape, dtype="bf16", device="cuda"):
    import torch

    dt = {"bf16": torch.bfloat16, "f32": torch.float32, "i64": torch.int64,
          "u8": torch.uint8, "fp8": torch.float8_e4m3fn}[dtype]
    return torch.zeros(shape, dtype=dt, device=device)


def test_norm_and_silu_refuse_mismatched_tensors(rra):
    say("[binding] norm / silu")
    x, w = _t(8, 512), _t(512)
    with pytest.raises(ValueError):  # residual with fewer rows than x
        rra.fused_add_rmsnorm_quant(x, _t(4, 512), w, 1e-6, 2)
    with pytest.raises(ValueError):  # output with fewer rows
        rra.fused_add_rmsnorm_quant(x, None, w, 1e-6, 2, out=_t(4, 512, dtype="fp8"))
    with pytest.raises(ValueError):  # per-group scales of the wrong shape
        rra.fused_add_rmsnorm_quant(x, None, w, 1e-6, 3, 128, scales=_t(8, 2, dtype="f32"))
    with pytest.raises(TypeError):  # static scale on the host
        rra.fused_add_rmsnorm_quant(x, None, w, 1e-6, 1, 0, _t(1, dtype="f32", device="cpu"))
    with pytest.raises(TypeError):  # static scale of the wrong type
        rra.fused_add_rmsnorm_quant(x, None, w, 1e-6, 1, 0, _t(1))
    with pytest.raises(ValueError):  # empty static scale
        rra.fused_add_rmsnorm_quant(x, None, w, 1e-6, 1, 0, _t(0, dtype="f32"))
    inp = _t(8, 1024)
    with pytest.raises(ValueError):  # odd gate|up width
        rra.silu_mul_quant(_t(8, 1025), 3, 128)
    with pytest.raises(ValueError):
        rra.silu_mul_quant(inp, 3, 128, out=_t(7, 512, dtype="fp8"))
    with pytest.raises(ValueError):
        rra.silu_mul_quant(inp, 3, 128, scales=_t(8, 3, dtype="f32"))


def test_rope_family_refuses_mismatched_tensors(rra):
    say("[binding] rope / qk norm / mla rope")
    T, Hq, Hkv, D = 6, 4, 2, 64
    q, k, v = _t(T, Hq, D), _t(T, Hkv, D), _t(T, Hkv, D)
    cs, kc, vc = _t(64, D, dtype="f32"), _t(4, 16, Hkv, D), _t(4, 16, Hkv, D)
    pos, slots = _t(T, dtype="i64"), _t(T, dtype="i64")
    with pytest.raises(ValueError):  # more positions than tokens
        rra.rope_kv_write(_t(T + 1, dtype="i64"), q, k, v, cs, slots, kc, vc)
    with pytest.raises(ValueError):  # slot mapping shorter than the tokens
        rra.rope_kv_write(pos, q, k, v, cs, _t(T - 1, dtype="i64"), kc, vc)
    with pytest.raises(ValueError):  # k with fewer tokens than q
        rra.rope_kv_write(pos, q, _t(T - 2, Hkv, D), v, cs, slots, kc, vc)
    with pytest.raises(ValueError):  # caches of different shapes
        rra.rope_kv_write(pos, q, k, v, cs, slots, kc, _t(2, 16, Hkv, D))
    with pytest.raises(ValueError):  # q_out with fewer tokens
        rra.rope_kv_write(pos, q, k, v, cs, slots, kc, vc, q_out=_t(T - 1, Hq, D))
    qkv = _t(T, (Hq + 2 * Hkv) * D)
    w = _t(D)
    with pytest.raises(ValueError):
        rra.qk_norm_rope_kv_write(_t(T + 3, dtype="i64"), qkv, w, w, 1e-6, cs, Hq, Hkv, D)
    with pytest.raises(ValueError):
        rra.qk_norm_rope_kv_write(pos, qkv, w, w, 1e-6, cs, Hq, Hkv, D,
                                  slot_mapping=_t(2, dtype="i64"), key_cache=kc, value_cache=vc)
    with pytest.raises(rra.RRAError):  # no cache and k not written back: k would be dropped
        rra.qk_norm_rope_kv_write(pos, qkv, w, w, 1e-6, cs, Hq, Hkv, D, write_k=False)
    mq = _t(T, 8 * 192)
    with pytest.raises(ValueError):  # k_pe with fewer tokens than q
        rra.mla_rope_kv_write(pos, mq, _t(T - 1, 64), _t(T, 512), cs, slots,
                              _t(4, 16, 576), 8, 64, 192, 128)
    with pytest.raises(ValueError):  # kv_c with fewer tokens
        rra.mla_rope_kv_write(pos, mq, _t(T, 64), _t(T - 1, 512), cs, slots,
                              _t(4, 16, 576), 8, 64, 192, 128)
    with pytest.raises(ValueError):  # table of another rope width
        rra.mla_rope_kv_write(pos, mq, _t(T, 64), _t(T, 512), _t(64, 128, dtype="f32"), slots,
                              _t(4, 16, 576), 8, 64, 192, 128)


def test_mla_norm_pad_and_encode_refuse_mismatched_tensors(rra):
    say("[binding] mla norm / pad / encode")
    q, kv, qw, kvw = _t(5, 1536), _t(5, 512), _t(1536), _t(512)
    with pytest.raises(ValueError):  # kv with fewer rows than q
        rra.dual_rmsnorm_quant(q, qw, 1e-6, _t(4, 512), kvw, 1e-6, 3, 128)
    with pytest.raises(ValueError):
        rra.dual_rmsnorm_quant(q, qw, 1e-6, kv, kvw, 1e-6, 3, 128, q_scales=_t(5, 6, dtype="f32"))
    with pytest.raises(ValueError):
        rra.dual_rmsnorm_quant(q, qw, 1e-6, kv, kvw, 1e-6, 3, 128, kv_out=_t(3, 512))
    x = _t(4, 2880)
    with pytest.raises(ValueError):
        rra.fused_add_rmsnorm_pad(x, _t(3, 2880), _t(2880), 1e-5, 3072)
    with pytest.raises(ValueError):
        rra.fused_add_rmsnorm_pad(x, None, _t(2880), 1e-5, 3072, out=_t(2, 3072))
    with pytest.raises(ValueError):
        rra.e4m3fn_encode(_t(16, dtype="f32"), out=_t(8, dtype="u8"))
