"""The C-ABI library: it loads, exports every function include/rra.h declares,
and rejects bad arguments on the host before anything is launched.

These tests make no compute call: every call below either fails validation
(NULL, misaligned or out-of-range arguments, with fake pointers that are never
dereferenced) or has T == 0, which returns before any HIP call."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rra.h")

OK, ENULL, ESHAPE, EALIGN, EUNSUP = 0, -1, -2, -3, -4
A = 0x10000  # a 16-byte aligned fake device address (never dereferenced)


@pytest.fixture(scope="module")
def rra():
    import rope_residual_add_amd as r

    if not os.path.exists(r.LIBRARY_PATH):
        from rope_residual_add_amd import build

        build.build()
    r.lib()
    return r


def declared_functions() -> list:
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("fused_add_rmsnorm_quant", "silu_mul_quant", "rope_kv_write", "dual_rmsnorm_quant",
              "qk_norm_rope_kv_write", "fused_add_rmsnorm_pad", "mla_rope_kv_write",
              "rope_cos_sin_cache", "rra_e4m3fn_encode", "rra_stream_copy", "rra_abi_version",
              "rra_status_string"):
        assert n in names


def test_library_exports_every_declared_function(rra):
    out = subprocess.run(["nm", "-D", "--defined-only", rra.LIBRARY_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
    assert set(rra.EXPORTS) == set(declared_functions())


def test_version_and_status_strings(rra):
    assert rra.abi_version() == rra.ABI_VERSION == 6
    for s in (OK, ENULL, ESHAPE, EALIGN, EUNSUP, -5):
        assert rra.status_string(s) and rra.status_string(s) != "unknown status"
    assert rra.status_string(-99) == "unknown status"


def norm(L, **kw):
    a = dict(x=A, xs=4096, res=A, rs=4096, w=A, eps=1e-5, mode=2, g=0, ss=None, out=A, os=4096,
             sc=A, T=4, H=4096)
    a.update(kw)
    return L.fused_add_rmsnorm_quant(a["x"], a["xs"], a["res"], a["rs"], a["w"], a["eps"],
                                     a["mode"], a["g"], a["ss"], a["out"], a["os"], a["sc"],
                                     a["T"], a["H"], None)


def test_norm_validation(rra):
    L = rra.lib()
    assert norm(L, T=0) == OK
    assert norm(L, x=None) == ENULL
    assert norm(L, sc=None) == ENULL  # per-token needs scales
    assert norm(L, mode=1, ss=None, T=0) == ENULL  # static needs the scale pointer
    assert norm(L, T=-1) == ESHAPE
    assert norm(L, xs=100) == ESHAPE
    assert norm(L, H=4100, xs=4104, rs=4104, os=4104) == EUNSUP  # H % 8
    assert norm(L, H=8200, xs=8200, rs=8200, os=8200) == EUNSUP  # above the register cap
    assert norm(L, mode=3, g=96) == EUNSUP
    assert norm(L, mode=3, g=128, H=4032, xs=4032, rs=4032, os=4032) == ESHAPE  # g does not divide H
    assert norm(L, mode=0) == EUNSUP
    assert norm(L, mode=7) == EUNSUP
    assert norm(L, x=A + 8) == EALIGN
    assert norm(L, xs=4100) == EALIGN
    assert norm(L, out=A + 4) == EALIGN
    assert norm(L, res=None, rs=0, T=0) == OK
    # with T == 0 the per-row tensors may be NULL (empty tensors), the weight may not
    assert norm(L, x=None, res=None, out=None, sc=None, T=0) == OK
    assert norm(L, w=None, T=0) == ENULL
    assert norm(L, T=(1 << 31) + 5) == EUNSUP  # one row per workgroup: grid above 2^31 - 1


def test_silu_validation(rra):
    L = rra.lib()
    f = lambda **k: L.silu_mul_quant(k.get("inp", A), k.get("s", 28672), k.get("mode", 3),
                                     k.get("g", 128), k.get("ss", None), k.get("out", A),
                                     k.get("os", 14336), k.get("sc", A), k.get("T", 2),
                                     k.get("I", 14336), None)
    assert f(T=0) == OK
    assert f(inp=None) == ENULL
    assert f(sc=None) == ENULL
    assert f(s=14336) == ESHAPE
    assert f(g=32) == EUNSUP
    assert f(mode=2) == EUNSUP  # per-token is not offered for this op
    assert f(I=1000, s=2000, os=1000) == ESHAPE  # 128 does not divide 1000
    assert f(inp=A + 2) == EALIGN
    assert f(mode=1, ss=None) == ENULL
    assert f(inp=None, out=None, sc=None, T=0) == OK
    # one wave per 512-column chunk (28 per row here): 2^31 waves or more are refused
    assert f(T=(1 << 31) // 28 + 1) == EUNSUP
    assert f(T=(1 << 31) + 1, I=512, s=1024, os=512) == EUNSUP
    assert f(I=1 << 62, s=1 << 62, os=1 << 62) == EUNSUP  # no overflow in the stride checks


def test_rope_validation(rra):
    L = rra.lib()

    def f(**k):
        a = dict(pos=A, q=A, qs=4096, qo=A, qos=4096, k=A, ks=1024, v=A, vs=1024, cs=A, mp=8192,
                 sm=A, kc=A, vc=A, T=4, Hq=32, Hkv=8, D=128, rd=128, bs=16, nb=4096, neox=1,
                 dt=rra.BF16)
        a.update(k)
        return L.rope_kv_write(a["pos"], a["q"], a["qs"], a["qo"], a["qos"], a["k"], a["ks"],
                               a["v"], a["vs"], a["cs"], a["mp"], a["sm"], a["kc"], a["vc"],
                               a["T"], a["Hq"], a["Hkv"], a["D"], a["rd"], a["bs"], a["nb"],
                               a["neox"], a["dt"], None)

    assert f(T=0) == OK
    assert f(sm=None) == ENULL
    assert f(qs=2048) == ESHAPE
    assert f(D=96, qs=3072, qos=3072, ks=768, vs=768, rd=96) == EUNSUP
    assert f(rd=64) == EUNSUP
    assert f(neox=2) == EUNSUP
    assert f(dt=2) == EUNSUP and f(dt=-1) == EUNSUP  # only bf16 and fp16
    assert f(dt=rra.F16, T=0) == OK
    assert f(dt=rra.F16, q=A + 2) == EALIGN  # fp16 keeps the 16-byte rules
    assert f(pos=None, q=None, qo=None, k=None, v=None, sm=None, T=0) == OK
    assert f(kc=None, T=0) == ENULL
    assert f(cs=None, T=0) == ENULL
    assert f(kc=A + 2) == EALIGN
    assert f(pos=A + 4) == EALIGN
    assert f(bs=0) == ESHAPE
    # the kernel carries the q and k token strides as 32-bit counts of 8 elements
    assert f(qs=8 << 32, T=0) == EUNSUP and f(ks=8 << 32, T=0) == EUNSUP
    assert f(qs=(8 << 32) - 8, ks=(8 << 32) - 8, T=0) == OK
    # six waves per token at this shape (384 units, one per lane): a launch of
    # 2^31 waves or more is refused before anything is enqueued
    assert f(T=(1 << 31) // 6 + 1) == EUNSUP
    assert f(T=(1 << 31) + 1, Hq=1, Hkv=1, qs=128, qos=128, ks=128, vs=128) == EUNSUP
    assert f(T=1 << 62) == EUNSUP  # refused before any product of T
    assert f(Hq=(1 << 16) + 1) == EUNSUP  # head counts up to 65536
    assert L.rope_cos_sin_cache(None, 8192, 128, 5e5, None) == ENULL
    assert L.rope_cos_sin_cache(A, 8192, 127, 5e5, None) == ESHAPE
    assert L.rope_cos_sin_cache(A, 8192, 128, -1.0, None) == EUNSUP
    assert L.rope_cos_sin_cache(A, 0, 128, 5e5, None) == OK


def test_dual_validation(rra):
    L = rra.lib()

    def f(**k):
        a = dict(q=A, qs=1536, qw=A, eq=1e-6, kv=A, kvs=512, kvw=A, ekv=1e-6, mode=3, g=128,
                 qo=A, qos=1536, sc=A, kvo=A, kvos=512, T=2, Hq=1536, Hkv=512)
        a.update(k)
        return L.dual_rmsnorm_quant(a["q"], a["qs"], a["qw"], a["eq"], a["kv"], a["kvs"],
                                    a["kvw"], a["ekv"], a["mode"], a["g"], a["qo"], a["qos"],
                                    a["sc"], a["kvo"], a["kvos"], a["T"], a["Hq"], a["Hkv"], None)

    assert f(T=0) == OK
    assert f(kvo=None) == ENULL
    assert f(q=None, kv=None, qo=None, kvo=None, sc=None, T=0) == OK
    assert f(qw=None, T=0) == ENULL
    assert f(sc=None) == ENULL
    assert f(mode=1) == EUNSUP
    assert f(Hq=4096, qs=4096, qos=4096) == EUNSUP
    assert f(kv=A + 8, T=0) == EALIGN  # alignment is checked before the T == 0 early return
    assert f(g=64, Hq=1000, qs=1000, qos=1000) == ESHAPE  # 64 does not divide 1000
    assert f(T=4 << 31) == EUNSUP  # four tokens per workgroup: grid above 2^31 - 1


def test_qk_norm_rope_validation(rra):
    L = rra.lib()

    def f(**k):
        a = dict(pos=A, qkv=A, s=6144, qw=A, kw=A, eps=1e-6, cs=A, mp=8192, sm=A, kc=A, vc=A,
                 wk=0, T=4, Hq=32, Hkv=8, D=128, rd=128, bs=16, nb=4096, neox=1)
        a.update(k)
        return L.qk_norm_rope_kv_write(a["pos"], a["qkv"], a["s"], a["qw"], a["kw"], a["eps"],
                                       a["cs"], a["mp"], a["sm"], a["kc"], a["vc"], a["wk"],
                                       a["T"], a["Hq"], a["Hkv"], a["D"], a["rd"], a["bs"],
                                       a["nb"], a["neox"], None)

    assert f(T=0) == OK
    assert f(pos=None, qkv=None, sm=None, kc=None, vc=None, wk=1, T=0) == OK
    # without a cache, k's result has only qkv to go to: write_k = 0 is refused
    assert f(sm=None, kc=None, vc=None, wk=0) == EUNSUP
    assert f(sm=None, kc=None, vc=None, wk=0, T=0) == EUNSUP
    assert f(qw=None, T=0) == ENULL
    assert f(kc=None) == ENULL  # a slot mapping needs both caches
    assert f(s=4096) == ESHAPE  # narrower than (Hq + 2 Hkv) D
    assert f(D=96, s=4608, rd=96) == EUNSUP
    assert f(rd=64) == EUNSUP
    assert f(neox=2) == EUNSUP
    assert f(qkv=A + 2) == EALIGN
    assert f(kw=A + 8) == EALIGN
    assert f(bs=0) == ESHAPE
    assert f(T=(1 << 31) // 6 + 1) == EUNSUP  # 384 units: six waves per token
    assert f(Hkv=70000) == EUNSUP


def test_rmsnorm_pad_validation(rra):
    L = rra.lib()

    def f(**k):
        a = dict(x=A, xs=2880, r=A, rs=2880, w=A, eps=1e-5, o=A, os=3072, T=4, H=2880, Hp=3072,
                 dt=rra.BF16)
        a.update(k)
        return L.fused_add_rmsnorm_pad(a["x"], a["xs"], a["r"], a["rs"], a["w"], a["eps"],
                                       a["o"], a["os"], a["T"], a["H"], a["Hp"], a["dt"], None)

    assert f(T=0) == OK
    assert f(x=None, r=None, o=None, T=0) == OK
    assert f(w=None, T=0) == ENULL
    assert f(Hp=2872) == ESHAPE  # pad narrower than H
    assert f(os=3000) == ESHAPE  # out row narrower than H_pad
    assert f(Hp=3076, os=3076) == EUNSUP  # H_pad % 8
    assert f(o=A + 8) == EALIGN
    assert f(x=A + 2) == EALIGN
    assert f(dt=2) == EUNSUP and f(dt=rra.F16, x=A + 2) == EALIGN
    assert f(dt=rra.F16, T=0) == OK


def test_mla_rope_validation(rra):
    L = rra.lib()

    def f(**k):
        a = dict(pos=A, q=A, qs=24576, hs=192, kpe=A, ks=64, c=A, cs_=512, cs=A, mp=8192, sm=A,
                 kv=A, T=4, Hq=128, lora=512, rd=64, bs=64, nb=1024, neox=0)
        a.update(k)
        return L.mla_rope_kv_write(a["pos"], a["q"], a["qs"], a["hs"], a["kpe"], a["ks"],
                                   a["c"], a["cs_"], a["cs"], a["mp"], a["sm"], a["kv"], a["T"],
                                   a["Hq"], a["lora"], a["rd"], a["bs"], a["nb"], a["neox"],
                                   None)

    assert f(T=0) == OK
    assert f(pos=None, q=None, kpe=None, c=None, sm=None, T=0) == OK
    assert f(kv=None, T=0) == ENULL
    assert f(qs=1000) == ESHAPE  # rows too narrow for 128 heads at stride 192
    assert f(hs=32) == ESHAPE  # head stride below rope_dim
    assert f(rd=32, ks=32) == EUNSUP
    assert f(lora=500, cs_=500) == EUNSUP
    assert f(neox=2) == EUNSUP
    assert f(T=(1 << 31) // 18 + 1) == EUNSUP  # 1096 one-vector units: eighteen waves per token
    assert f(Hq=70000) == EUNSUP
    assert f(hs=1 << 62) == ESHAPE  # (Hq - 1) * head stride past the row, without overflow
    assert f(hs=196, qs=25088) == EALIGN  # head stride not a multiple of 8
    assert f(kv=A + 4) == EALIGN
    # the kernel carries the q_pe strides as 32-bit counts of 8 elements
    assert f(qs=8 << 32, T=0) == EUNSUP
    assert f(qs=(8 << 32) - 8, T=0) == OK
    assert f(Hq=1, hs=8 << 32, T=0) == EUNSUP  # one head: its stride is otherwise unbounded


def test_e4m3_diag_validation(rra):
    L = rra.lib()
    assert L.rra_e4m3fn_encode(None, A, 4, None) == ENULL
    assert L.rra_e4m3fn_encode(A + 4, A, 4, None) == EALIGN
    assert L.rra_e4m3fn_encode(A, A, 0, None) == OK


def test_stream_copy_validation(rra):
    L = rra.lib()
    assert L.rra_stream_copy(None, A + 4096, 16, 1, None) == ENULL
    assert L.rra_stream_copy(A, None, 16, 1, None) == ENULL
    assert L.rra_stream_copy(A, A + 4096, -16, 1, None) == ESHAPE
    assert L.rra_stream_copy(A, A + 4096, 24, 1, None) == EALIGN  # not a whole number of vectors
    assert L.rra_stream_copy(A + 8, A + 4096, 16, 1, None) == EALIGN
    assert L.rra_stream_copy(A, A + 4104, 16, 1, None) == EALIGN
    assert L.rra_stream_copy(A, A + 16, 32, 1, None) == ESHAPE  # overlapping ranges
    assert L.rra_stream_copy(A + 16, A, 32, 1, None) == ESHAPE
    assert L.rra_stream_copy(A, A + 4096, 16, 3, None) == EUNSUP  # vectors per lane
    assert L.rra_stream_copy(A, A + 4096, 16, 16, None) == EUNSUP
    assert L.rra_stream_copy(None, None, 0, 1, None) == OK
