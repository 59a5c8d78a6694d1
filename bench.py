#!/usr/bin/env python3
"""Throughput of the four fused kernels on one MI355X.

One step is one pass over the whole fused path at T tokens (default 8192):
  fused_add_rmsnorm_quant  residual add + RMSNorm + per-token FP8, hidden 4096 (Llama-3-8B)
  silu_mul_quant           SiLU-and-Mul + per-group-128 FP8, intermediate 14336 (Llama-3-8B)
  rope_kv_write            neox RoPE (32 q / 8 kv heads of 128, theta 5e5) + paged KV write
                           into a [4096, 16, 8, 128] bf16 cache through a slot mapping
  dual_rmsnorm_quant       MLA q (1536, per-group-128 FP8) / kv (512, bf16) RMSNorm (DeepSeek-V3)
on seeded synthetic inputs already resident in HBM.  The step streams about
1.1 GB, several times the 256 MB last-level cache, so every kernel starts on
cold data.  The K timed steps follow --settle-ms of untimed steps and then the
W warm-up steps, so that they run at the clocks the GPU holds under sustained
load; "settle" also reports the same K steps timed straight after set-up.

Bandwidth is counted in ALGORITHMIC bytes: each input read once and each
output written once (per token: 7H + 4 for the norm, 5I + 4I/128 for SiLU,
24592 for RoPE + KV write, 6704 for the MLA norm; plus the weights once per
launch).  Per-kernel durations come from HIP events (created without a system
fence) recorded on the stream the kernels run on, around every launch of the
timed region.

Prints ONE JSON line on stdout (everything else goes to stderr).  Beside the
step it reports, each timed alone and cold (rotating buffer sets) next to a
streaming copy of the same bytes: the next-row kernels ("next_rows"), the
other quantization modes ("modes": static and per-group-128 norm, static
SiLU), and the fusion's effect ("fusion": fused against unfused bytes, and the
MLA norm's two-launch form timed against its one launch), and the step at
decode-size token counts launched one by one against replayed from a HIP graph
("decode").  "target" lists the
kernels at or below 75% of peak HBM bandwidth; "cpu_baseline" times the
oracle.  With --sweep it also times each kernel alone at several token counts
and adds the table under "sweep".
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E peak
TARGET_FRAC = 0.75  # the bar: each kernel at >= 75% of peak HBM bandwidth
METRIC = "achieved HBM GB/s (% of MI355X peak) and tokens/s per fused kernel, T=8192"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---- algorithmic bytes ---------------------------------------------------------

H_NORM, I_SILU, G = 4096, 14336, 128
ROPE_HQ, ROPE_HKV, ROPE_D = 32, 8, 128
MLA_HQ, MLA_HKV = 1536, 512

BYTES_PER_TOKEN = {
    "fused_add_rmsnorm_quant": 7 * H_NORM + 4,
    "silu_mul_quant": 5 * I_SILU + 4 * (I_SILU // G),
    "rope_kv_write": 2 * 2 * ROPE_HQ * ROPE_D + 2 * 2 * ROPE_HKV * ROPE_D + 2 * 2 * ROPE_HKV * ROPE_D
    + 16,
    "dual_rmsnorm_quant": 2 * MLA_HQ + 2 * MLA_HKV + MLA_HQ + 4 * (MLA_HQ // G) + 2 * MLA_HKV,
}
BYTES_PER_LAUNCH = {  # weights, read once per launch
    "fused_add_rmsnorm_quant": 2 * H_NORM,
    "silu_mul_quant": 0,
    "rope_kv_write": 0,
    "dual_rmsnorm_quant": 2 * (MLA_HQ + MLA_HKV),
}
KERNELS = tuple(BYTES_PER_TOKEN)

# The next rows, measured beside the step (not part of it): QK norm + RoPE + KV
# write at the Qwen3-8B attention shape, residual add + RMSNorm + padding at
# GPT-OSS width, MLA q_pe/k_pe RoPE + [kv_c | k_pe] cache write at DeepSeek-V3,
# and the RoPE + KV write of the step and the padding op with fp16 instead of
# bf16 elements.
QK_HQ, QK_HKV, QK_D = 32, 8, 128
PAD_H, PAD_HP = 2880, 3072
MR_HQ, MR_NOPE, MR_ROPE, MR_LORA = 128, 128, 64, 512
BYTES_PER_TOKEN.update({
    "rope_kv_write_f16": BYTES_PER_TOKEN["rope_kv_write"],
    "fused_add_rmsnorm_pad_f16": 2 * 2 * PAD_H + 2 * PAD_H + 2 * PAD_HP,
    "qk_norm_rope_kv_write": 2 * (QK_HQ + 2 * QK_HKV) * QK_D + 2 * QK_HQ * QK_D
    + 2 * 2 * QK_HKV * QK_D + 16,
    "fused_add_rmsnorm_pad": 2 * 2 * PAD_H + 2 * PAD_H + 2 * PAD_HP,
    "mla_rope_kv_write": 2 * 2 * MR_HQ * MR_ROPE + 2 * MR_ROPE + 2 * MR_LORA
    + 2 * (MR_LORA + MR_ROPE) + 16,
})
BYTES_PER_LAUNCH.update({
    "rope_kv_write_f16": 0,
    "fused_add_rmsnorm_pad_f16": 2 * PAD_H,
    "qk_norm_rope_kv_write": 2 * 2 * QK_D,
    "fused_add_rmsnorm_pad": 2 * PAD_H,
    "mla_rope_kv_write": 0,
})
NEXT_KERNELS = ("qk_norm_rope_kv_write", "fused_add_rmsnorm_pad", "mla_rope_kv_write",
                "rope_kv_write_f16", "fused_add_rmsnorm_pad_f16")

# The other quantization modes the pages list, timed beside the step (not part
# of it): the residual-add norm with a static scale at the small config's width
# (H = 1024, eps 1e-6, scale 0.05) and with per-group-128 scales at the
# Llama-3-8B width, and SiLU-and-Mul with a static scale.
H_STATIC = 1024
BYTES_PER_TOKEN.update({
    "fused_add_rmsnorm_quant_static": 7 * H_STATIC,
    "fused_add_rmsnorm_quant_g128": 7 * H_NORM + 4 * (H_NORM // G),
    "silu_mul_quant_static": 5 * I_SILU,
})
BYTES_PER_LAUNCH.update({
    "fused_add_rmsnorm_quant_static": 2 * H_STATIC + 4,
    "fused_add_rmsnorm_quant_g128": 2 * H_NORM,
    "silu_mul_quant_static": 4,
})
MODE_KERNELS = ("fused_add_rmsnorm_quant_static", "fused_add_rmsnorm_quant_g128",
                "silu_mul_quant_static")

# Bytes the unfused form of each pattern moves per token (the pages' "without
# the fusion" pipelines, each step reading its inputs and writing its outputs):
#   norm: fused_add_rms_norm (x, residual in; residual and a bf16 y out), then
#         the quant (y in; codes and the scale out): 11H + 4;
#   SiLU: silu_and_mul (gate|up in, bf16 activation out), then the quant: 9I + 4I/128;
#   RoPE: rotary (q, k and the position in; q and k out), then the cache write
#         (k, v and the slot in; both cache rows out);
#   MLA norm: the same bytes as the fused op, in two launches.
UNFUSED_BYTES_PER_TOKEN = {
    "fused_add_rmsnorm_quant": 11 * H_NORM + 4,
    "silu_mul_quant": 9 * I_SILU + 4 * (I_SILU // G),
    "rope_kv_write": 2 * 2 * ROPE_HQ * ROPE_D + 2 * 2 * ROPE_HKV * ROPE_D + 8
    + 2 * 2 * ROPE_HKV * ROPE_D + 2 * 2 * ROPE_HKV * ROPE_D + 8,
    "dual_rmsnorm_quant": BYTES_PER_TOKEN["dual_rmsnorm_quant"],
}


def algo_bytes(name: str, T: int) -> int:
    return BYTES_PER_TOKEN[name] * T + BYTES_PER_LAUNCH[name]


# Work-items per launch at T tokens, as the library launches these workloads
# (used only to tell the sweep's launches apart in a kernel trace):
#  - residual-add norms: up to 1024 rows, one vector per lane and one row per
#    workgroup of max(4, waves per row) waves (H = 4096: 8 waves; H = 1024: two
#    rows of 2 waves); above, four waves per row at widths above 2048 (one
#    workgroup per row), one wave per row up to 1024 (four rows per workgroup);
#  - SiLU: one wave per 512 outputs;
#  - MLA norm: up to 1024 tokens one workgroup of 4 waves per token (one wave
#    per 512-column vector at 1536 / 512), above one wave per token;
#  - the RoPE family: as many waves per token as its units need at one unit per
#    lane (Llama-3-8B / Qwen3-8B attention: 48 heads x 8 two-vector units, six
#    waves; DeepSeek-V3 MLA: 129 heads x 8 one-vector units + 64 kv_c vectors,
#    eighteen).
NORM_SPLIT_MAX_T, DUAL_SPLIT_MAX_T = 1024, 1024


def _rope_waves_per_token(units: int) -> int:
    ku = max(1, -(-units // 2048))
    return -(-(-(-units // ku)) // 64)


def _norm_shape(T: int, H: int) -> tuple:
    """(vectors per lane, waves per row) of the residual-add norms' launch."""
    need = -(-H // 512)
    if T <= NORM_SPLIT_MAX_T:
        return 1, next(w for w in (1, 2, 4, 8, 16) if w >= need)
    kw = 1 if H <= 1024 else (2 if H <= 2048 else 4)
    return -(-H // (512 * kw)), kw


def _norm_threads(T: int, H: int) -> int:
    _, kw = _norm_shape(T, H)
    block_waves = max(4, kw)
    return 64 * block_waves * -(-T // (block_waves // kw))


def launch_symbol(name: str, T: int):
    """A fragment of the demangled symbol the library launches for the kernel
    at T, where its launch shape depends on T (the decode-size shapes), so that
    trace rows of equal grid size but different shape are told apart; None
    where one symbol serves every T."""
    if name == "dual_rmsnorm_quant":
        return ("rra::dual_rmsnorm_split_kernel<" if T <= DUAL_SPLIT_MAX_T
                else "rra::dual_rmsnorm_quant_kernel<")
    H = {"fused_add_rmsnorm_quant": H_NORM, "fused_add_rmsnorm_quant_g128": H_NORM,
         "fused_add_rmsnorm_quant_static": H_STATIC, "fused_add_rmsnorm_pad": PAD_H,
         "fused_add_rmsnorm_pad_f16": PAD_H}.get(name)
    if H is None:
        return None
    nv, kw = _norm_shape(T, H)
    sym = "add_rmsnorm_pad_kernel" if "pad" in name else "add_rmsnorm_quant_kernel"
    return f"rra::{sym}<{nv}, {kw}, "


def grid_threads(name: str, T: int) -> int:
    import workloads

    if name in ("silu_mul_quant", "silu_mul_quant_static"):
        waves = T * -(-I_SILU // 512)
    elif name in ("rope_kv_write", "rope_kv_write_f16"):
        cfg = workloads.ROPE
        units = (cfg.Hq + 2 * cfg.Hkv) * (cfg.D // 16 if cfg.is_neox else cfg.D // 8)
        waves = T * _rope_waves_per_token(units)
    elif name == "qk_norm_rope_kv_write":
        cfg = workloads.QKNORM
        waves = T * _rope_waves_per_token((cfg.Hq + 2 * cfg.Hkv) * (cfg.D // 16))
    elif name == "mla_rope_kv_write":
        cfg = workloads.MLA_ROPE
        per_head = cfg.rope_dim // 16 if cfg.is_neox else cfg.rope_dim // 8
        waves = T * _rope_waves_per_token((cfg.Hq + 1) * per_head + cfg.kv_lora // 8)
    elif name == "dual_rmsnorm_quant":
        return 256 * T if T <= DUAL_SPLIT_MAX_T else 256 * -(-T // 4)
    elif name == "fused_add_rmsnorm_quant_static":
        return _norm_threads(T, H_STATIC)
    elif name in ("fused_add_rmsnorm_pad", "fused_add_rmsnorm_pad_f16"):
        return _norm_threads(T, PAD_H)
    else:
        return _norm_threads(T, H_NORM)
    return 64 * 4 * -(-waves // 4)


def copy_half_bytes(nbytes_moved: int) -> int:
    """Bytes read (= bytes written) by the same-size copy yardstick."""
    return max(16, (nbytes_moved // 2) // 16 * 16)


# ---- kernel identity: symbols and sources ----------------------------------------

CSRC = os.path.join(ROOT, "rope_residual_add_amd", "csrc")
# The demangled kernel names of each measured kernel: symbol and the template
# arguments that tell modes and element types apart (quant mode 1 static, 2
# per token, 3 per group; rows of the MLA norm take its one-wave-per-token or
# its decode-size kernel).
KERNEL_NAME_RE = {
    "fused_add_rmsnorm_quant": r"rra::add_rmsnorm_quant_kernel<\d+, \d+, true, 2, 0, \w+>",
    "fused_add_rmsnorm_quant_static": r"rra::add_rmsnorm_quant_kernel<\d+, \d+, true, 1, 0, \w+>",
    "fused_add_rmsnorm_quant_g128": r"rra::add_rmsnorm_quant_kernel<\d+, \d+, true, 3, 128, \w+>",
    "silu_mul_quant": r"rra::silu_mul_quant_kernel<3, 128, \w+>",
    "silu_mul_quant_static": r"rra::silu_mul_quant_kernel<1, 0, \w+>",
    "rope_kv_write": r"rra::rope_kv_write_kernel<\d+, \w+, \d+, rra::ElemBf16>",
    "rope_kv_write_f16": r"rra::rope_kv_write_kernel<\d+, \w+, \d+, rra::ElemF16>",
    "dual_rmsnorm_quant": r"rra::dual_rmsnorm_(quant|split)_kernel<",
    "qk_norm_rope_kv_write": r"rra::qk_norm_rope_kv_kernel<",
    "fused_add_rmsnorm_pad": r"rra::add_rmsnorm_pad_kernel<\d+, \d+, true, \w+, rra::ElemBf16>",
    "fused_add_rmsnorm_pad_f16": r"rra::add_rmsnorm_pad_kernel<\d+, \d+, true, \w+, rra::ElemF16>",
    "mla_rope_kv_write": r"rra::mla_rope_kv_kernel<",
}
KERNEL_SOURCES = {
    "fused_add_rmsnorm_quant": ("norm_quant.hip",),
    "fused_add_rmsnorm_quant_static": ("norm_quant.hip",),
    "fused_add_rmsnorm_quant_g128": ("norm_quant.hip",),
    "silu_mul_quant_static": ("silu_mul_quant.hip",),
    "dual_rmsnorm_quant": ("norm_quant.hip",),
    "silu_mul_quant": ("silu_mul_quant.hip",),
    "rope_kv_write": ("rope_kv.hip",),
    "qk_norm_rope_kv_write": ("rope_kv.hip",),
    "fused_add_rmsnorm_pad": ("norm_quant.hip",),
    "mla_rope_kv_write": ("rope_kv.hip",),
    "rope_kv_write_f16": ("rope_kv.hip",),
    "fused_add_rmsnorm_pad_f16": ("norm_quant.hip",),
}
COMMON_SOURCES = ("rra_device.hpp", "rra_host.hpp")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "fused_kernels_T8192_hbm_traffic.md")


def _code_only(text: str) -> str:
    """C++ source with comments removed and whitespace runs collapsed (string
    literals in these sources hold no comment markers)."""
    import re

    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(kernel: str) -> str:
    """sha256 (first 16 hex digits) of the code of the sources a kernel is
    built from (comments and layout excluded), so that stored counter readings
    can be matched to the code they measured."""
    import hashlib

    h = hashlib.sha256()
    for name in sorted(KERNEL_SOURCES[kernel] + COMMON_SOURCES):
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str):
    """HBM bytes per launch from the committed counter summary, or None when
    the summary is missing or the kernel's sources changed since."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    want = source_hash(kernel)
    for line in text.splitlines():
        cells = [c.strip().strip("`") for c in line.strip().strip("|").split("|")]
        if len(cells) >= 7 and cells[0] == kernel and cells[1] == want:
            return int(cells[5])
    return None


# ---- HIP events ----------------------------------------------------------------------
# Kernel durations are taken with HIP events recorded on the stream the kernels
# run on (torch's current stream, which the binding hands to the library).  The
# events are created with hipEventDisableSystemFence: a timing marker then needs
# no system-scope release, which otherwise adds 1-3 us to every bracketed
# launch.  The HIP runtime is the one torch has loaded (same soname).

class HipEvents:
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes

        self._c = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                     ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        for f in ("hipEventCreateWithFlags", "hipEventRecord", "hipEventElapsedTime",
                  "hipEventDestroy"):
            getattr(self.hip, f).restype = ctypes.c_int

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def create(self, n: int) -> list:
        out = []
        for _ in range(n):
            e = self._c.c_void_p()
            self._ok(self.hip.hipEventCreateWithFlags(self._c.byref(e), self.DISABLE_SYSTEM_FENCE),
                     "hipEventCreateWithFlags")
            out.append(e)
        return out

    def record(self, e, stream) -> None:
        self._ok(self.hip.hipEventRecord(e, self._c.c_void_p(stream)), "hipEventRecord")

    def ms(self, a, b) -> float:
        v = self._c.c_float()
        self._ok(self.hip.hipEventElapsedTime(self._c.byref(v), a, b), "hipEventElapsedTime")
        return v.value

    def destroy(self, evs) -> None:
        for e in evs:
            self.hip.hipEventDestroy(e)


# ---- GPU side ------------------------------------------------------------------

def make_launchers(T: int, salt: int = 0, shared=None, only=KERNELS):
    """Allocate one input/output set at T tokens for each kernel in `only` and
    return {name: zero-argument launch function}.  L["_shared"] holds, per
    cache-writing kernel, its cache(s) and cos/sin table; passing that dict as
    `shared` makes further buffer sets reuse them."""
    import torch

    import rope_residual_add_amd as rra
    import workloads

    dev = "cuda"
    L = {}
    io = {}  # every kernel's tensors, for checking the timed launch path
    L["_io"] = io
    shared = dict(shared or {})
    L["_shared"] = shared

    if "fused_add_rmsnorm_quant" in only:
        d = workloads.device_norm_inputs(T, H_NORM, dev, salt)
        out = torch.empty((T, H_NORM), dtype=torch.float8_e4m3fn, device=dev)
        sc = torch.empty((T,), dtype=torch.float32, device=dev)
        L["fused_add_rmsnorm_quant"] = lambda d=d, out=out, sc=sc: rra.fused_add_rmsnorm_quant(
            d["x"], d["residual"], d["weight"], 1e-5, rra.Q_PER_TOKEN, 0, None, out, sc)
        io["fused_add_rmsnorm_quant"] = dict(d, out=out, scales=sc)

    if "silu_mul_quant" in only:
        d = workloads.device_silu_inputs(T, I_SILU, dev, salt)
        out = torch.empty((T, I_SILU), dtype=torch.float8_e4m3fn, device=dev)
        sc = torch.empty((T, I_SILU // G), dtype=torch.float32, device=dev)
        L["silu_mul_quant"] = lambda d=d, out=out, sc=sc: rra.silu_mul_quant(
            d["inp"], rra.Q_PER_GROUP, G, None, out, sc)
        io["silu_mul_quant"] = dict(d, out=out, scales=sc)

    if "rope_kv_write" in only:
        cfg = workloads.ROPE
        state = shared.get("rope_kv_write")
        d = workloads.device_rope_inputs(T, cfg, dev, salt, with_cache=state is None)
        if state is None:
            cs = rra.rope_cos_sin_cache(cfg.max_pos, cfg.rot_dim, cfg.theta, device=dev)
            state = shared["rope_kv_write"] = (d["key_cache"], d["value_cache"], cs)
        kc, vc, cs = state
        L["rope_kv_write"] = lambda d=d, kc=kc, vc=vc, cs=cs: rra.rope_kv_write(
            d["positions"], d["q"], d["k"], d["v"], cs, d["slot_mapping"], kc, vc)
        io["rope_kv_write"] = dict(d, key_cache=kc, value_cache=vc)

    if "rope_kv_write_f16" in only:
        cfg = workloads.ROPE_F16
        state = shared.get("rope_kv_write_f16")
        d = workloads.device_rope_inputs(T, cfg, dev, salt, with_cache=state is None)
        if state is None:
            cs = rra.rope_cos_sin_cache(cfg.max_pos, cfg.rot_dim, cfg.theta, device=dev)
            state = shared["rope_kv_write_f16"] = (d["key_cache"], d["value_cache"], cs)
        kc, vc, cs = state
        L["rope_kv_write_f16"] = lambda d=d, kc=kc, vc=vc, cs=cs: rra.rope_kv_write(
            d["positions"], d["q"], d["k"], d["v"], cs, d["slot_mapping"], kc, vc)
        io["rope_kv_write_f16"] = dict(d, key_cache=kc, value_cache=vc)

    if "qk_norm_rope_kv_write" in only:
        cfg = workloads.QKNORM
        state = shared.get("qk_norm_rope_kv_write")
        d = workloads.device_qknorm_inputs(T, cfg, dev, salt, with_cache=state is None)
        if state is None:
            cs_q = rra.rope_cos_sin_cache(cfg.max_pos, cfg.D, cfg.theta, device=dev)
            state = shared["qk_norm_rope_kv_write"] = (d["key_cache"], d["value_cache"], cs_q)
        kc, vc, cs_q = state
        def qkn(d=d, kc=kc, vc=vc, cs=cs_q, cfg=cfg):
            return rra.qk_norm_rope_kv_write(
                d["positions"], d["qkv"], d["q_w"], d["k_w"], cfg.eps, cs, cfg.Hq, cfg.Hkv,
                cfg.D, slot_mapping=d["slot_mapping"], key_cache=kc, value_cache=vc)
        L["qk_norm_rope_kv_write"] = qkn
        io["qk_norm_rope_kv_write"] = dict(d, key_cache=kc, value_cache=vc)

    for name, cfg in (("fused_add_rmsnorm_pad", workloads.PAD),
                      ("fused_add_rmsnorm_pad_f16", workloads.PAD_F16)):
        if name not in only:
            continue
        d = workloads.device_pad_inputs(T, cfg, dev, salt)
        out = torch.empty((T, cfg.H_pad), dtype=d["x"].dtype, device=dev)
        L[name] = lambda d=d, out=out, cfg=cfg: rra.fused_add_rmsnorm_pad(
            d["x"], d["residual"], d["weight"], cfg.eps, cfg.H_pad, out)
        io[name] = dict(d, out=out)

    if "mla_rope_kv_write" in only:
        cfg = workloads.MLA_ROPE
        state = shared.get("mla_rope_kv_write")
        d = workloads.device_mla_rope_inputs(T, cfg, dev, salt, with_cache=state is None)
        if state is None:
            cs_m = rra.rope_cos_sin_cache(cfg.max_pos, cfg.rope_dim, cfg.theta, device=dev)
            state = shared["mla_rope_kv_write"] = (d["kv_cache"], cs_m)
        cache, cs_m = state
        L["mla_rope_kv_write"] = lambda d=d, cache=cache, cs=cs_m, cfg=cfg: rra.mla_rope_kv_write(
            d["positions"], d["q"], d["k_pe"], d["kv_c"], cs, d["slot_mapping"], cache, cfg.Hq,
            cfg.rope_dim, cfg.nope + cfg.rope_dim, cfg.nope, is_neox=cfg.is_neox)
        io["mla_rope_kv_write"] = dict(d, kv_cache=cache)

    if "fused_add_rmsnorm_quant_static" in only:
        d = workloads.device_norm_inputs(T, H_STATIC, dev, salt)
        sc0 = torch.full((1,), 0.05, dtype=torch.float32, device=dev)
        out = torch.empty((T, H_STATIC), dtype=torch.float8_e4m3fn, device=dev)
        L["fused_add_rmsnorm_quant_static"] = lambda d=d, out=out, sc0=sc0: (
            rra.fused_add_rmsnorm_quant(d["x"], d["residual"], d["weight"], 1e-6, rra.Q_STATIC,
                                        0, sc0, out))
        io["fused_add_rmsnorm_quant_static"] = dict(d, out=out, static_scale=sc0)

    if "fused_add_rmsnorm_quant_g128" in only:
        d = workloads.device_norm_inputs(T, H_NORM, dev, salt)
        out = torch.empty((T, H_NORM), dtype=torch.float8_e4m3fn, device=dev)
        sc = torch.empty((T, H_NORM // G), dtype=torch.float32, device=dev)
        L["fused_add_rmsnorm_quant_g128"] = lambda d=d, out=out, sc=sc: (
            rra.fused_add_rmsnorm_quant(d["x"], d["residual"], d["weight"], 1e-5,
                                        rra.Q_PER_GROUP, G, None, out, sc))
        io["fused_add_rmsnorm_quant_g128"] = dict(d, out=out, scales=sc)

    if "silu_mul_quant_static" in only:
        d = workloads.device_silu_inputs(T, I_SILU, dev, salt)
        sc0 = torch.full((1,), 0.05, dtype=torch.float32, device=dev)
        out = torch.empty((T, I_SILU), dtype=torch.float8_e4m3fn, device=dev)
        L["silu_mul_quant_static"] = lambda d=d, out=out, sc0=sc0: rra.silu_mul_quant(
            d["inp"], rra.Q_STATIC, 0, sc0, out)
        io["silu_mul_quant_static"] = dict(d, out=out, static_scale=sc0)

    if "dual_rmsnorm_quant" in only:
        d = workloads.device_mla_inputs(T, workloads.MLA, dev, salt)
        qo = torch.empty((T, MLA_HQ), dtype=torch.float8_e4m3fn, device=dev)
        qs = torch.empty((T, MLA_HQ // G), dtype=torch.float32, device=dev)
        kvo = torch.empty((T, MLA_HKV), dtype=torch.bfloat16, device=dev)
        L["dual_rmsnorm_quant"] = lambda d=d, qo=qo, qs=qs, kvo=kvo: rra.dual_rmsnorm_quant(
            d["q"], d["q_w"], 1e-6, d["kv"], d["kv_w"], 1e-6, rra.Q_PER_GROUP, G, qo, qs, kvo)
        io["dual_rmsnorm_quant"] = dict(d, q_out=qo, q_scales=qs, kv_out=kvo)
    torch.cuda.synchronize()
    return L


def _timed_pass(launch, steps: int, warmup: int) -> float:
    """`warmup` untimed steps, then the wall time of `steps` steps, each timed
    region bracketed by a device synchronization."""
    import torch

    for _ in range(warmup):
        for n in KERNELS:
            launch[n]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        for n in KERNELS:
            launch[n]()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def settle(launch, ms: float) -> int:
    """Untimed steps until the GPU has run them for at least `ms` milliseconds.
    An MI355X raises its clocks only under sustained load: the first ~10 ms of
    steps after an idle spell run about 4% slower than the steady state.
    Returns the number of steps run."""
    import torch

    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(20):
            for k in KERNELS:
                launch[k]()
        n += 20
        torch.cuda.synchronize()
    return n


def run_steps(launch, steps: int, warmup: int, settle_ms: float = 0.0):
    """Time `steps` passes over the four kernels (launch: the dict of
    make_launchers), three ways:
      - from idle: `warmup` steps, then `steps` timed, straight after set-up;
      - steady: untimed steps for `settle_ms` (settle), `warmup` steps, then
        `steps` timed, for the whole step's wall time at loaded clocks;
      - per kernel: HIP events around every launch, queued behind a spin
        kernel, for each kernel's duration.
    Returns (steady wall seconds, from-idle wall seconds, settle steps,
    {kernel: [per-launch ms]})."""
    import torch

    idle_wall = _timed_pass(launch, steps, warmup)
    settled = settle(launch, settle_ms) if settle_ms > 0 else 0
    wall = _timed_pass(launch, steps, warmup)

    hip = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    nk = len(KERNELS)
    ev = hip.create(steps * (nk + 1))
    # All launches and events of the pass are queued behind a spin kernel
    # (long enough for the host to issue them, ~15 us each), so that each
    # interval holds the GPU's own time between two launches and never a
    # wait for the host.
    cyc = _blocker_cycles(max(5.0, 0.03 * steps * (2 * nk + 1)))
    torch.cuda.synchronize()
    torch.cuda._sleep(cyc)
    for s in range(steps):
        base = s * (nk + 1)
        hip.record(ev[base], stream)
        for i, n in enumerate(KERNELS):
            launch[n]()
            hip.record(ev[base + i + 1], stream)
    torch.cuda.synchronize()
    per = {n: [hip.ms(ev[s * (nk + 1) + i], ev[s * (nk + 1) + i + 1]) for s in range(steps)]
           for i, n in enumerate(KERNELS)}
    hip.destroy(ev)
    return wall, idle_wall, settled, per


def _blocker_cycles(target_ms: float = 5.0) -> int:
    """Spin-kernel length (torch.cuda._sleep cycles) that keeps the GPU busy
    for about target_ms, so that launches queued behind it run back to back
    and the events around them time the kernels, not the host's launch rate."""
    import torch

    probe = 1_000_000
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    torch.cuda._sleep(probe)
    b.record()
    torch.cuda.synchronize()
    ms = max(a.elapsed_time(b), 1e-3)
    return int(min(probe * target_ms / ms, 2_000_000_000))


def copy_ceiling(nbytes: int = 1 << 30, n_pairs: int = 4, reps: int = 12) -> dict:
    """The library's streaming copy (same 16-byte loads and stores, same cache
    policy as the fused kernels) of nbytes, rotating over n_pairs of buffers
    (8 GiB in all) so that it streams from HBM: read + write bytes / time."""
    import torch

    import rope_residual_add_amd as rra

    src = [torch.full((nbytes,), i + 1, dtype=torch.uint8, device="cuda") for i in range(n_pairs)]
    dst = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(n_pairs)]
    for i in range(n_pairs):
        rra.stream_copy(src[i], dst[i])
    cyc = _blocker_cycles()
    hip = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    ev = hip.create(2)
    torch.cuda._sleep(cyc)
    hip.record(ev[0], stream)
    for r in range(reps):
        rra.stream_copy(src[r % n_pairs], dst[r % n_pairs])
    hip.record(ev[1], stream)
    torch.cuda.synchronize()
    ms = hip.ms(ev[0], ev[1]) / reps
    hip.destroy(ev)
    gbps = 2 * nbytes / (ms * 1e-3) / 1e9
    log(f"copy ceiling: {nbytes >> 20} MiB stream copy {ms * 1e3:.1f} us -> {gbps:.1f} GB/s "
        f"({100 * gbps / PEAK_HBM_GBPS:.1f}% of 8 TB/s)")
    del src, dst
    torch.cuda.empty_cache()
    return dict(gbps=round(gbps, 1), frac_of_peak=round(gbps / PEAK_HBM_GBPS, 4),
                what=f"rra_stream_copy of {nbytes >> 20} MiB (read + write bytes), {n_pairs} "
                     f"rotating buffer pairs, {reps} launches back to back")


def _timed_launches(hip, stream, cyc, fns, n: int) -> float:
    """Median ms of n launches, fns[j % len(fns)] for launch j, each bracketed
    by events and all queued behind a spin kernel."""
    import torch

    ev = hip.create(2 * n)
    torch.cuda._sleep(cyc)  # queue the timed launches behind a spin kernel
    for j in range(n):
        hip.record(ev[2 * j], stream)
        fns[j % len(fns)]()
        hip.record(ev[2 * j + 1], stream)
    torch.cuda.synchronize()
    ms = statistics.median(hip.ms(ev[2 * j], ev[2 * j + 1]) for j in range(n))
    hip.destroy(ev)
    return ms


COPY_VECTORS_PER_LANE = (1, 2, 4, 8)


def copy_yardstick(nbytes_moved: int, launches: int, hip, stream, cyc):
    """(median ms, vectors per lane) of the fastest streaming copy that moves
    nbytes_moved bytes in all (half read, half written), cold, timed like the
    sweep's kernels; the copy is tried with 1, 2, 4 and 8 vectors per lane,
    whose best choice changes with the size."""
    import torch

    import rope_residual_add_amd as rra

    half = copy_half_bytes(nbytes_moved)
    n_sets = max(2, min(256, -(-(1 << 30) // (2 * half))))
    bufs = [(torch.empty(half, dtype=torch.uint8, device="cuda"),
             torch.empty(half, dtype=torch.uint8, device="cuda")) for _ in range(n_sets)]
    best = None
    for v in COPY_VECTORS_PER_LANE:
        fns = [lambda a=a, b=b, v=v: rra.stream_copy(a, b, v) for a, b in bufs]
        for f in fns:
            f()
        torch.cuda.synchronize()
        ms = _timed_launches(hip, stream, cyc, fns, launches)
        if best is None or ms < best[0]:
            best = (ms, v)
    del bufs
    torch.cuda.empty_cache()
    return best


# Timed launches per sweep point (after one warm-up launch per buffer set).
SWEEP_LAUNCHES = 30


def sweep(Ts, launches_per_point: int = SWEEP_LAUNCHES, kernels=KERNELS, with_copy: bool = True):
    """Each kernel alone at each T, rotating over buffer sets of that kernel
    that total at least 1 GiB of algorithmic traffic (four times the 256 MB
    last-level cache), so every launch reads cold data.  With with_copy, each
    point is also compared with the library's streaming copy moving the same
    number of bytes (half read, half written), timed the same way: the
    achievable rate at that size, launch and ramp included."""
    import torch

    rows = []
    cyc = _blocker_cycles()
    hip = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    for T in Ts:
        for n in kernels:
            n_sets = max(2, min(256, -(-(1 << 30) // algo_bytes(n, T))))
            sets = []
            shared = None  # one cache (and table) shared by the kernel's buffer sets
            for salt in range(n_sets):
                L = make_launchers(T, salt, shared, only=(n,))
                shared = L["_shared"]
                sets.append(L)
            for s in sets:  # warm-up: one launch per set
                s[n]()
            torch.cuda.synchronize()
            ms = _timed_launches(hip, stream, cyc, [s[n] for s in sets], launches_per_point)
            del sets
            torch.cuda.empty_cache()
            b = algo_bytes(n, T)
            gbps = b / (ms * 1e-3) / 1e9
            row = dict(kernel=n, T=T, us=round(ms * 1e3, 2), gbps=round(gbps, 1),
                       frac=round(gbps / PEAK_HBM_GBPS, 4),
                       tokens_per_s=round(T / (ms * 1e-3), 1), buffer_sets=n_sets)
            if with_copy:
                cms, cv = copy_yardstick(b, launches_per_point, hip, stream, cyc)
                row.update(copy_us=round(cms * 1e3, 2), copy_vectors_per_lane=cv,
                           frac_of_copy=round(cms / ms, 4))
            rows.append(row)
            log(f"sweep {n:26s} T={T:6d} {ms * 1e3:9.2f} us {gbps:8.1f} GB/s "
                f"({100 * gbps / PEAK_HBM_GBPS:5.1f}% of peak), {n_sets} buffer sets"
                + (f"; same-size copy {row['copy_us']:8.2f} us ({100 * row['frac_of_copy']:5.1f}%)"
                   if with_copy else ""))
    return rows


def back_to_back(T: int, kernels=KERNELS, launches: int = 40) -> dict:
    """Each kernel alone at T, `launches` launches queued back to back behind a
    spin kernel with one event pair around them all, rotating over buffer sets
    of that kernel holding at least 1 GiB (every launch reads cold data):
    {kernel: average ms per launch}.  Unlike an event pair around every launch,
    this adds no event between launches, so the average is the kernel's own
    duration plus the gap the hardware leaves between two queued kernels: the
    way the copy ceiling is timed."""
    import torch

    out = {}
    cyc = _blocker_cycles()
    hip = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    for n in kernels:
        n_sets = max(2, min(256, -(-(1 << 30) // algo_bytes(n, T))))
        sets, shared = [], None
        for salt in range(n_sets):
            L = make_launchers(T, salt, shared, only=(n,))
            shared = L["_shared"]
            sets.append(L)
        for s in sets:  # warm-up: one launch per set
            s[n]()
        torch.cuda.synchronize()
        ev = hip.create(2)
        torch.cuda._sleep(cyc)
        hip.record(ev[0], stream)
        for j in range(launches):
            sets[j % n_sets][n]()
        hip.record(ev[1], stream)
        torch.cuda.synchronize()
        out[n] = hip.ms(ev[0], ev[1]) / launches
        hip.destroy(ev)
        del sets
        torch.cuda.empty_cache()
        b = algo_bytes(n, T)
        log(f"back to back {n:26s} T={T:6d} {out[n] * 1e3:9.2f} us "
            f"{b / (out[n] * 1e-3) / 1e9:8.1f} GB/s, {n_sets} buffer sets")
    return out


def dual_two_launch(Ts, launches: int = 60) -> dict:
    """The MLA norm as the pages' unfused form runs it, two launches (q: RMSNorm
    + per-group-128 FP8 quant with fused_add_rmsnorm_quant and no residual; kv:
    RMSNorm to bf16 with fused_add_rmsnorm_pad and no padding), against the
    one-launch dual_rmsnorm_quant, at each T: median of event intervals around
    the one launch or the pair, queued behind a spin kernel, cold (rotating
    buffer sets of at least 1 GiB, at most 256).  Both forms move the same
    bytes; the difference is the second launch."""
    import torch

    import rope_residual_add_amd as rra
    import workloads

    cyc = _blocker_cycles()
    hip = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    for T in Ts:
        b = algo_bytes("dual_rmsnorm_quant", T)
        n_sets = max(2, min(256, -(-(1 << 30) // b)))
        sets = []
        for salt in range(n_sets):
            d = workloads.device_mla_inputs(T, workloads.MLA, "cuda", salt)
            sets.append((d, torch.empty((T, MLA_HQ), dtype=torch.float8_e4m3fn, device="cuda"),
                         torch.empty((T, MLA_HQ // G), dtype=torch.float32, device="cuda"),
                         torch.empty((T, MLA_HKV), dtype=torch.bfloat16, device="cuda")))

        def one(d, qo, qs, kvo):
            rra.dual_rmsnorm_quant(d["q"], d["q_w"], 1e-6, d["kv"], d["kv_w"], 1e-6,
                                   rra.Q_PER_GROUP, G, qo, qs, kvo)

        def two(d, qo, qs, kvo):
            rra.fused_add_rmsnorm_quant(d["q"], None, d["q_w"], 1e-6, rra.Q_PER_GROUP, G, None,
                                        qo, qs)
            rra.fused_add_rmsnorm_pad(d["kv"], None, d["kv_w"], 1e-6, MLA_HKV, kvo)

        # the two forms give the same outputs (scales can differ in the last bit
        # only where a sum of squares is added in another order)
        for f in (one, two):
            for a in sets:
                f(*a)
        torch.cuda.synchronize()
        ref = [t.clone() for t in sets[0][1:]]
        two(*sets[0])
        torch.cuda.synchronize()
        same = dict(q_codes=int((ref[0].view(torch.uint8) != sets[0][1].view(torch.uint8))
                                .sum().item()),
                    q_scales=int((ref[1] != sets[0][2]).sum().item()),
                    kv=int((ref[2].view(torch.int16) != sets[0][3].view(torch.int16)).sum().item()))
        ms1 = _timed_launches(hip, stream, cyc, [lambda a=a: one(*a) for a in sets], launches)
        ms2 = _timed_launches(hip, stream, cyc, [lambda a=a: two(*a) for a in sets], launches)
        out[str(T)] = dict(one_launch_us=round(ms1 * 1e3, 2), two_launch_us=round(ms2 * 1e3, 2),
                           saved_us=round((ms2 - ms1) * 1e3, 2), bytes=b,
                           outputs_differing=same)
        log(f"MLA norm T={T}: one launch {ms1 * 1e3:.2f} us, two launches {ms2 * 1e3:.2f} us "
            f"(differing outputs {same})")
        del sets
        torch.cuda.empty_cache()
    return out


def decode_steps(Ts, steps: int = 200, per_graph: int = 10) -> dict:
    """The step's four kernels at decode-size token counts, timed per step two
    ways: launched one by one through the binding (its host cost included, as
    an eager serving loop pays it) and replayed from a HIP graph captured over
    `per_graph` steps (torch.cuda.CUDAGraph; the library allocates nothing and
    only enqueues, so its calls capture as they are).  After the timed
    replays, the outputs that each step rewrites from unchanged inputs (SiLU's
    codes, the key cache, the MLA norm's q codes and scales) are checked
    against the eager ones.  Returns
    {T: {eager_us_per_step, graph_us_per_step, outputs_equal}}."""
    import torch

    rows = {}
    for T in Ts:
        launch = make_launchers(T, salt=5)

        def step():
            for n in KERNELS:
                launch[n]()

        for _ in range(5):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        eager = (time.perf_counter() - t0) / steps
        # Outputs that every step rewrites from unchanged inputs (the norm's
        # residual and RoPE's q are updated in place, so theirs move on).
        io = launch["_io"]
        outs = [io["silu_mul_quant"]["out"], io["rope_kv_write"]["key_cache"],
                io["dual_rmsnorm_quant"]["q_out"], io["dual_rmsnorm_quant"]["q_scales"]]
        eager_out = [o.clone() for o in outs]
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                for _ in range(per_graph):
                    step()
        torch.cuda.current_stream().wait_stream(side)
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // per_graph)
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        replayed = (time.perf_counter() - t0) / (reps * per_graph)
        same = all(torch.equal(a.view(torch.uint8), b.view(torch.uint8))
                   for a, b in zip(outs, eager_out))
        rows[str(T)] = dict(eager_us_per_step=round(eager * 1e6, 2),
                            graph_us_per_step=round(replayed * 1e6, 2), outputs_equal=same)
        log(f"decode T={T}: {eager * 1e6:.1f} us per step launched one by one, "
            f"{replayed * 1e6:.1f} us replayed from a graph (outputs equal: {same})")
        del graph, launch
    return rows


def fusion_report(kern: dict, T: int, dual: dict) -> dict:
    """Fused against unfused bytes per launch at T, with the unfused form's
    time projected at the fused kernel's own measured bandwidth (the unfused
    kernels are not part of this library), and the MLA norm's measured one- and
    two-launch times."""
    rep = {}
    for k in ("fused_add_rmsnorm_quant", "silu_mul_quant", "rope_kv_write"):
        fused = algo_bytes(k, T)
        unfused = UNFUSED_BYTES_PER_TOKEN[k] * T + BYTES_PER_LAUNCH[k]
        rep[k] = dict(fused_bytes=fused, unfused_bytes=unfused,
                      unfused_over_fused=round(unfused / fused, 4), fused_us=kern[k]["us"],
                      unfused_us_projected=round(kern[k]["us"] * unfused / fused, 2))
    rep["dual_rmsnorm_quant"] = dict(fused_bytes=algo_bytes("dual_rmsnorm_quant", T),
                                     unfused_bytes=algo_bytes("dual_rmsnorm_quant", T),
                                     launches_measured=dual)
    rep["note"] = ("unfused_us_projected = fused time x unfused/fused bytes (the fused kernel's "
                   "own bandwidth); the MLA norm's two-launch form is measured")
    return rep


def environment() -> dict:
    """Versions and device facts recorded beside the numbers."""
    import platform

    import torch

    p = torch.cuda.get_device_properties(0)
    cpu_model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            names = [ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")]
        cpu_model = names[0] if names else cpu_model
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return dict(device=torch.cuda.get_device_name(0), arch=getattr(p, "gcnArchName", ""),
                compute_units=p.multi_processor_count, memory_gib=round(p.total_memory / 2**30, 1),
                torch=torch.__version__, hip=getattr(torch.version, "hip", None),
                host_cpus=os.cpu_count(), host_cpus_usable=usable, host_cpu=cpu_model)


# ---- CPU baseline: the oracle on a bounded sample --------------------------------

def _oracle_call(name: str, n: int):
    """Zero-argument oracle call on n tokens of a kernel's workload."""
    import oracle
    import workloads

    if name in ("fused_add_rmsnorm_quant", "fused_add_rmsnorm_quant_g128"):
        d = workloads.norm_inputs(n, H_NORM)
        mode, g = ((oracle.Q_PER_TOKEN, 0) if name == "fused_add_rmsnorm_quant"
                   else (oracle.Q_PER_GROUP, G))
        return lambda: oracle.fused_add_rmsnorm_quant(d["x"], d["residual"], d["weight"], 1e-5,
                                                      mode, g)
    if name == "fused_add_rmsnorm_quant_static":
        d = workloads.norm_inputs(n, H_STATIC)
        return lambda: oracle.fused_add_rmsnorm_quant(d["x"], d["residual"], d["weight"], 1e-6,
                                                      oracle.Q_STATIC, 0, 0.05)
    if name in ("silu_mul_quant", "silu_mul_quant_static"):
        d = workloads.silu_inputs(n, I_SILU)
        if name == "silu_mul_quant":
            return lambda: oracle.silu_mul_quant(d["inp"], oracle.Q_PER_GROUP, G)
        return lambda: oracle.silu_mul_quant(d["inp"], oracle.Q_STATIC, 0, 0.05)
    if name == "rope_kv_write":
        cfg = workloads.ROPE
        d = workloads.rope_inputs(n, cfg)
        return lambda: oracle.rope_kv_write(
            d["positions"], d["q"], d["k"], d["v"], cfg.theta, cfg.max_pos, d["slot_mapping"],
            d["key_cache"], d["value_cache"], cfg.Hq, cfg.Hkv, cfg.D)
    if name == "dual_rmsnorm_quant":
        d = workloads.mla_inputs(n)
        return lambda: oracle.dual_rmsnorm_quant(d["q"], d["q_w"], 1e-6, d["kv"], d["kv_w"], 1e-6,
                                                 oracle.Q_PER_GROUP, G)
    raise KeyError(name)


# Each config's largest token count beside the step's T (the RoPE and MLA
# configs go to 16384), and the other quantization modes at the step's T.
ORACLE_LARGEST_T = {"rope_kv_write": 16384, "dual_rmsnorm_quant": 16384}
ORACLE_REPS = 5


def cpu_baseline(T: int, one_core_T: int = 1024) -> dict:
    """The oracle as it stands, timed on the host's cores (up to 16): the GPU
    step's own workload at T tokens, each config's largest T, and the other
    quantization modes at T; plus one core on one_core_T tokens.  One warm-up,
    then the median of five calls each.  Reported in GB/s of the same
    algorithmic bytes as the GPU, with tokens/s per kernel."""
    import oracle

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, 16))

    def timed(name, n, threads):
        f = _oracle_call(name, n)
        oracle.set_threads(threads)
        f()  # warm-up
        ts = []
        for _ in range(ORACLE_REPS):
            t0 = time.perf_counter()
            f()
            ts.append(time.perf_counter() - t0)
        sec = statistics.median(ts)
        log(f"oracle {name:32s} T={n:6d} {sec * 1e3:8.1f} ms on {oracle.get_threads()} threads")
        return sec, int(oracle.get_threads())

    def point(name, n, sec):
        b = algo_bytes(name, n)
        return dict(T=n, ms=round(sec * 1e3, 2), gbps=round(b / sec / 1e9, 4),
                    tokens_per_s=round(n / sec, 1))

    def summary(n, secs):
        total_bytes = sum(algo_bytes(k, n) for k in KERNELS)
        return dict(value=round(total_bytes / sum(secs.values()) / 1e9, 4), unit="GB/s",
                    per_kernel_ms={k: round(v * 1e3, 2) for k, v in secs.items()},
                    tokens_per_s={k: round(n / v, 1) for k, v in secs.items()})

    one = {k: timed(k, one_core_T, 1)[0] for k in KERNELS}
    secs, used = {}, 1
    for k in KERNELS:
        secs[k], used = timed(k, T, cores)
    out = summary(T, secs)
    out.update(cores=used, kind="oracle",
               sample=f"the GPU step's workload, T={T} tokens of each of the four kernels; "
                      f"fp64 C oracle, OpenMP over rows, median of {ORACLE_REPS} calls after "
                      f"one warm-up; bytes counted as for the GPU; largest_T: the RoPE and MLA "
                      f"configs at T=16384; modes: the other quantization modes at T={T}; "
                      f"one_core: T={one_core_T} on one thread. The RoPE oracle returns fresh "
                      f"copies of both 128 MiB caches on every call, which is a large part of "
                      f"its time")
    out["largest_T"] = {k: point(k, n, timed(k, n, cores)[0])
                        for k, n in ORACLE_LARGEST_T.items()}
    out["modes"] = {k: point(k, T, timed(k, T, cores)[0]) for k in MODE_KERNELS}
    out["one_core"] = dict(summary(one_core_T, one), T=one_core_T)
    return out


# ---- profile summaries (rocprofv3 CSV -> profiles/*.md) ----------------------------

def _kernel_of(symbol_name: str):
    """The measured kernel a demangled kernel name belongs to, or None."""
    import re

    for k, pat in KERNEL_NAME_RE.items():
        if re.search(pat, symbol_name):
            return k
    return None


def _launch_of(symbol_name: str, grid_items: int, T: int):
    """The measured kernel a dispatch belongs to when it ran that kernel's
    workload at T tokens (its grid has grid_threads(kernel, T) work-items), or
    None.  Other launches of the same symbol (the MLA norm's decode-size
    timings, a different T) are left out."""
    k = _kernel_of(symbol_name)
    if k is None or grid_items != grid_threads(k, T):
        return None
    frag = launch_symbol(k, T)
    return k if frag is None or frag in symbol_name else None


def summarize_trace(stats_csv: str, out: str, command: str, T: int, bench_json=None) -> None:
    """Kernel-trace summary of a traced bench run: per kernel, the profiler's
    durations of its launches at T (average, min, max, p10 / median / p90, from
    the per-dispatch trace next to the stats file, launches told apart by grid
    size) and GB/s; with bench_json (the JSON line the traced run printed), the
    run's own event-timed average per kernel beside the profiler's."""
    import collections
    import csv

    per = collections.defaultdict(list)
    sym = {}
    trace_csv = stats_csv.replace("kernel_stats", "kernel_trace")
    for r in csv.DictReader(open(trace_csv)):
        k = _launch_of(r["Kernel_Name"], int(r["Grid_Size_X"]), T)
        if k is not None and k in KERNELS:
            per[k].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
            sym[k] = r["Kernel_Name"].split("(")[0].replace("void ", "")
    events, b2b = {}, {}
    if bench_json:
        line = [ln for ln in open(bench_json).read().splitlines() if ln.startswith("{")][-1]
        kern = json.loads(line)["kernels"]
        events = {k: v["us"] for k, v in kern.items()}
        b2b = {k: v["back_to_back"]["us"] for k, v in kern.items() if "back_to_back" in v}

    lines = [f"# Kernel trace: the four fused kernels at T={T}", "",
             "Produced by (from the repository root, after `cd /tmp && export TMPDIR=/tmp` for "
             "the profiler):", "", "```", command, "```", "",
             "Durations are the profiler's kernel times of every launch of each kernel at "
             f"T={T} in the traced run (the step's passes: from idle, the settle steps, the timed "
             "steps and the event-timed steps; the back-to-back launches of each kernel alone; "
             "for the MLA norm also the one-launch side of the bench's two-launch comparison; "
             "launches told apart by grid size). "
             "GB/s = algorithmic bytes per launch / average."
             + (" `bench.py events avg us` is the traced run's own mean of the event pairs "
                "around each launch of its timed steps" if events else "")
             + ("; `bench.py back-to-back us` its average over 40 launches of the kernel alone "
                "between one event pair." if b2b else ("." if events else "")), "",
             "| kernel | symbol | calls | avg us | min us | max us | p10 / median / p90 us | "
             "algorithmic bytes | GB/s (avg) | % of 8 TB/s |"
             + (" bench.py events avg us |" if events else "")
             + (" bench.py back-to-back us |" if b2b else ""),
             "|---|---|---|---|---|---|---|---|---|---|" + ("---|" if events else "")
             + ("---|" if b2b else "")]
    for k in KERNELS:
        d = per.get(k)
        if not d:
            continue
        avg = statistics.fmean(d)
        b = algo_bytes(k, T)
        gbps = b / avg
        q = statistics.quantiles(d, n=10) if len(d) > 1 else [avg, avg]
        lines.append(f"| {k} | `{sym[k]}` | {len(d)} | {avg / 1e3:.2f} | {min(d) / 1e3:.2f} | "
                     f"{max(d) / 1e3:.2f} | {q[0] / 1e3:.2f} / {statistics.median(d) / 1e3:.2f} / "
                     f"{q[-1] / 1e3:.2f} | {b} | {gbps:.0f} | {100 * gbps / PEAK_HBM_GBPS:.1f}% |"
                     + (f" {events[k]:.2f} |" if events else "")
                     + (f" {b2b[k]:.2f} |" if b2b else ""))
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_traffic(fetch_csv: str, write_csv: str, out: str, commands: str, T: int) -> None:
    """HBM traffic per launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    scaled by what the same counters read for the library's streaming copy of
    1 GiB in the bench's copy ceiling (read and written bytes known)."""
    import collections
    import csv

    def load(path, counter):
        d = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            if "rra::stream_copy_kernel" in name:
                d[name].append(float(r["Counter_Value"]))
            elif _launch_of(name, int(r["Grid_Size"]), T) is not None:
                d[name, "at T"].append(float(r["Counter_Value"]))
        return d

    fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    copy = [n for n in fetch if isinstance(n, str) and "rra::stream_copy_kernel" in n]
    if not copy:
        raise SystemExit("no streaming copy in the counter run")
    gib_kib = float(1 << 20)
    f_copy = statistics.median(v for v in fetch[copy[0]] if v > 0.4 * gib_kib)
    w_copy = statistics.median(v for v in write[copy[0]] if v > 0.4 * gib_kib)
    f_scale, w_scale = gib_kib / f_copy, gib_kib / w_copy
    lines = [f"# HBM traffic per launch at T={T} (rocprofv3 counters)", "",
             "Produced by (from the repository root):", "", "```", commands, "```", "",
             f"Scale factors from the library's streaming copy (`{copy[0].split('(')[0]}`) moving "
             f"1 GiB in the same runs: FETCH_SIZE reads {f_copy:.0f} KiB for 1 GiB read "
             f"(x{f_scale:.4f}), WRITE_SIZE reads {w_copy:.0f} KiB for 1 GiB written "
             f"(x{w_scale:.4f}).", "",
             "`source` is the hash of the kernel's source code (comments and layout "
             "excluded) when the counters were taken (bench.py reports `traffic` only while "
             "it matches).", "",
             "| kernel | source | FETCH_SIZE KiB | WRITE_SIZE KiB | launches | traffic bytes | "
             "algorithmic bytes | traffic / algorithmic |", "|---|---|---|---|---|---|---|---|"]
    for k in KERNELS + NEXT_KERNELS:
        names = [n for n in fetch if isinstance(n, tuple) and _kernel_of(n[0]) == k]
        if not names:
            continue
        fv = [v for n in names for v in fetch[n]]
        wv = [v for n in names for v in write[n]]
        fk, wk = statistics.median(fv), statistics.median(wv)
        traffic = int(round((fk * f_scale + wk * w_scale) * 1024))
        b = algo_bytes(k, T)
        lines.append(f"| {k} | `{source_hash(k)}` | {fk:.0f} | {wk:.0f} | {len(fv)} | {traffic} | "
                     f"{b} | {traffic / b:.4f} |")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


WAVE_COUNTERS = ("SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY",
                 "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU")


def summarize_waves(counter_csv: str, out: str, command: str, T: int) -> None:
    """Per-wave instruction and cycle counters (one rocprofv3 --pmc pass of the
    eight SQ counters in WAVE_COUNTERS) per kernel at T: VALU instructions per
    wave, and how a wave's cycles split between waiting on data or
    dependencies (SQ_WAIT_ANY), waiting for an issue slot (SQ_WAIT_INST_ANY)
    and issuing (SQ_ACTIVE_INST_ANY); the VALU time per SIMD is instructions x
    4 cycles (a wave64 instruction on a 16-lane SIMD) x waves / 1024 SIMDs at
    2.4 GHz.  `source` hashes the kernel's code as in the traffic summary."""
    import collections
    import csv

    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(counter_csv)):
        name = r["Kernel_Name"]
        k = ("copy (1 vector per lane)" if "rra::stream_copy_kernel<1>" in name
             else _launch_of(name, int(r["Grid_Size"]), T))
        if k is None:
            continue
        vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = [f"# Per-wave counters at T={T} (rocprofv3 --pmc, SQ block)", "",
             "Produced by (from the repository root, after `cd /tmp && export TMPDIR=/tmp` for "
             "the profiler):", "", "```", command, "```", "",
             f"Medians over the run's launches of each kernel at T={T} (told apart by grid "
             "size). Cycles per wave: `waiting on data` "
             "= SQ_WAIT_ANY (waiting on memory or a dependency), `waiting for issue` = "
             "SQ_WAIT_INST_ANY, `issuing` = SQ_ACTIVE_INST_ANY. VALU time per SIMD = VALU per "
             "wave x 4 cycles x waves / 1024 SIMDs / 2.4 GHz. `source` is the hash of the "
             "kernel's code (comments and layout excluded) when the counters were taken.", "",
             "| kernel | source | launches | waves | VALU / wave | VALU time per SIMD us | "
             "wave cycles | waiting on data | waiting for issue | issuing |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    order = [k for k in KERNELS + MODE_KERNELS + NEXT_KERNELS if k in vals]
    order += [k for k in vals if k not in order]
    for k in order:
        c = vals[k]
        if not c.get("SQ_WAVES"):
            continue
        m = {n: statistics.median(v) for n, v in c.items()}
        w = m["SQ_WAVES"]
        per = {n: m.get(n, 0.0) / w for n in WAVE_COUNTERS}
        cyc = per["SQ_WAVE_CYCLES"] or 1.0
        valu_us = per["SQ_INSTS_VALU"] * 4 * w / 1024 / 2.4e3
        src = f"`{source_hash(k)}`" if k in KERNEL_SOURCES else "-"
        lines.append(
            f"| {k} | {src} | {len(c['SQ_WAVES'])} | {w:.0f} | {per['SQ_INSTS_VALU']:.0f} | "
            f"{valu_us:.1f} | {cyc:.0f} | {per['SQ_WAIT_ANY']:.0f} "
            f"({100 * per['SQ_WAIT_ANY'] / cyc:.0f}%) | {per['SQ_WAIT_INST_ANY']:.0f} "
            f"({100 * per['SQ_WAIT_INST_ANY'] / cyc:.0f}%) | {per['SQ_ACTIVE_INST_ANY']:.0f} |")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_sweep(trace_csv: str, out: str, command: str, Ts, kernels=KERNELS) -> None:
    """Sweep summary from a rocprofv3 kernel trace of `bench.py --sweep-only`:
    per kernel and T, the median profiler duration of its launches (told apart
    by grid size), against the median of the same-size streaming copy."""
    import collections
    import csv

    import re

    dur = collections.defaultdict(list)  # (kernel or ("copy", V), grid work-items) -> ns
    launches = collections.defaultdict(list)  # (kernel, grid) -> [(symbol, ns)]
    for r in csv.DictReader(open(trace_csv)):
        name = r["Kernel_Name"]
        m = re.search(r"rra::stream_copy_kernel<(\d+)>", name)
        k = ("copy", int(m.group(1))) if m else _kernel_of(name)
        if k is None:
            continue
        ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        dur[(k, int(r["Grid_Size_X"]))].append(ns)
        launches[(k, int(r["Grid_Size_X"]))].append((name, ns))

    def copy_best(nbytes_moved):
        """(median ns, vectors per lane) of the fastest copy of that size."""
        n16 = copy_half_bytes(nbytes_moved) // 16
        best = None
        for v in COPY_VECTORS_PER_LANE:
            d = dur.get((("copy", v), 256 * -(-n16 // (256 * v))))
            if d and (best is None or statistics.median(d) < best[0]):
                best = (statistics.median(d), v)
        return best

    lines = ["# Kernel trace: each fused kernel alone, cold, across token counts", "",
             "Produced by (from the repository root, after `cd /tmp && export TMPDIR=/tmp` for "
             "the profiler):", "", "```", command, "```", "",
             "Each point rotates over buffer sets holding at least 1 GiB, so every launch reads "
             "cold data. Durations are the profiler's (median over the point's launches: one "
             "warm-up launch per buffer set, which the host issues one at a time with the GPU "
             "otherwise idle, then the timed launches, queued behind a spin kernel with an event "
             f"pair around each, {SWEEP_LAUNCHES} of them). Where `launches` exceeds "
             f"{2 * SWEEP_LAUNCHES}, the warm-up launches are most of them, and the median is "
             "the duration of an isolated launch: queued back to back with events between them, "
             "any kernel of a few microseconds, the copy included, reads about 3.5 us in the "
             "profiler. "
             "`copy` is the fastest of the library's streaming copies (`rra_stream_copy`, the "
             "fused kernels' own loads and stores, with 1, 2, 4 or 8 vectors per lane: `vpl`) "
             "moving the same number of bytes, half read and half written, timed the same way; "
             "`% of copy` = copy time / kernel time.", "",
             "| kernel | T | launches | median us | GB/s | % of 8 TB/s | tokens/s | copy us (vpl) | "
             "% of copy |", "|---|---|---|---|---|---|---|---|---|"]
    for T in Ts:
        for k in kernels:
            frag = launch_symbol(k, T)
            d = [ns for name, ns in launches.get((k, grid_threads(k, T)), ())
                 if frag is None or frag in name]
            if not d:
                continue
            med = statistics.median(d)
            b = algo_bytes(k, T)
            c = copy_best(b)
            lines.append(f"| {k} | {T} | {len(d)} | {med / 1e3:.2f} | {b / med:.0f} | "
                         f"{100 * b / med / PEAK_HBM_GBPS:.1f}% | {T / (med * 1e-9):.3g} | "
                         + (f"{c[0] / 1e3:.2f} ({c[1]}) | {100 * c[0] / med:.1f}% |" if c
                            else "- | - |"))
    floor = dur.get((("copy", 1), 256))
    if floor:
        lines += ["", f"One-workgroup copy (launch floor), profiler median: "
                      f"{statistics.median(floor) / 1e3:.2f} us over {len(floor)} launches."]
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ---- main ------------------------------------------------------------------------

def _sweep_kernels(args) -> tuple:
    names = tuple(k for k in args.sweep_kernels.split(",") if k)
    unknown = [k for k in names if k not in BYTES_PER_TOKEN]
    if unknown:
        raise SystemExit(f"unknown kernels for --sweep-kernels: {unknown}")
    return names


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed steps for this long before the warmup, so that the timed "
                         "steps run at the clocks the GPU holds under sustained load")
    ap.add_argument("--T", type=int, default=8192, help="tokens per step")
    ap.add_argument("--cpu-sample", type=int, default=8192,
                    help="tokens per kernel for the oracle baseline (0 = skip)")
    ap.add_argument("--sweep", default="", help="comma-separated token counts for the "
                                                "per-kernel cold-cache sweep")
    ap.add_argument("--next-rows", type=int, default=1,
                    help="1 = also time the next-row kernels alone at T (cold, rotating sets)")
    ap.add_argument("--modes", type=int, default=1,
                    help="1 = also time the other quantization modes alone at T (static and "
                         "per-group-128 norm, static SiLU)")
    ap.add_argument("--decode", default="1,16,64",
                    help="token counts at which the step is also timed launched one by one "
                         "and replayed from a HIP graph (empty = skip)")
    ap.add_argument("--fusion", type=int, default=1,
                    help="1 = also report fused against unfused bytes and time the MLA norm's "
                         "two-launch form against its one launch")
    ap.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV",
                    help="write a profiles/ summary from a rocprofv3 --stats run and exit")
    ap.add_argument("--sweep-kernels", default=",".join(KERNELS),
                    help="comma-separated kernels for --sweep / --summarize-sweep "
                         "(default: the four step kernels)")
    ap.add_argument("--sweep-only", action="store_true",
                    help="run only the --sweep (no step, ceiling or baseline): for profiling")
    ap.add_argument("--summarize-sweep", metavar="KERNEL_TRACE_CSV",
                    help="write a profiles/ summary of a traced --sweep-only run and exit")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write a profiles/ summary from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-waves", metavar="COUNTER_CSV",
                    help="write a profiles/ summary of a rocprofv3 --pmc run of the SQ wave "
                         "counters and exit")
    ap.add_argument("--out", help="output file for --summarize-*")
    ap.add_argument("--bench-json", help="with --summarize-trace: the traced run's JSON output")
    ap.add_argument("--command", default="", help="command line recorded in the summary")
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, args.command, args.T, args.bench_json)
        return 0
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.out, args.command, args.T)
        return 0
    if args.summarize_waves:
        summarize_waves(args.summarize_waves, args.out, args.command, args.T)
        return 0
    if args.summarize_sweep:
        summarize_sweep(args.summarize_sweep, args.out, args.command,
                        [int(t) for t in args.sweep.split(",") if t], _sweep_kernels(args))
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the four kernels are row-independent and "
              f"need no exchange, so --gpus {args.gpus} has nothing further to show here.",
              file=sys.stderr)
        return 2

    import torch

    import rope_residual_add_amd as rra

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        return 1
    rra.lib()  # fail loudly if the HIP library is missing
    T = args.T
    if args.sweep_only:
        rows = sweep([int(t) for t in args.sweep.split(",") if t], kernels=_sweep_kernels(args))
        hip = HipEvents()
        copy_yardstick(8192, 30, hip, torch.cuda.current_stream().cuda_stream, _blocker_cycles())
        print(json.dumps(dict(sweep=rows)), flush=True)
        return 0
    log(f"device: {torch.cuda.get_device_name(0)}; T={T}; steps={args.steps}; "
        f"warmup={args.warmup}")
    launch = make_launchers(T)
    wall, idle_wall, settled, per = run_steps(launch, args.steps, args.warmup, args.settle_ms)

    kern = {}
    for n in KERNELS:
        ms = statistics.fmean(per[n])
        b = algo_bytes(n, T)
        gbps = b / (ms * 1e-3) / 1e9
        q = statistics.quantiles(per[n], n=10) if len(per[n]) > 1 else [ms, ms]
        frac = gbps / PEAK_HBM_GBPS
        kern[n] = dict(us=round(ms * 1e3, 2), us_median=round(statistics.median(per[n]) * 1e3, 2),
                       us_p10=round(q[0] * 1e3, 2), us_p90=round(q[-1] * 1e3, 2),
                       bytes=b, gbps=round(gbps, 1), frac_of_peak=round(frac, 4),
                       meets_target=frac >= TARGET_FRAC, tokens_per_s=round(T / (ms * 1e-3), 1))
        log(f"{n:26s} {ms * 1e3:9.2f} us  {gbps:8.1f} GB/s  "
            f"{100 * frac:5.1f}% of 8 TB/s  {T / (ms * 1e-3):.3e} tokens/s  "
            f"{'meets' if frac >= TARGET_FRAC else 'misses'} the {100 * TARGET_FRAC:.0f}% target")

    step_bytes = sum(algo_bytes(n, T) for n in KERNELS)
    ms_per_step = wall / args.steps * 1e3
    value = step_bytes / (wall / args.steps) / 1e9
    dom = max(KERNELS, key=lambda n: kern[n]["us"])
    roofline = dict(bound="hbm", kernel=dom, achieved=kern[dom]["gbps"], peak=PEAK_HBM_GBPS,
                    unit="GB/s", frac=kern[dom]["frac_of_peak"], traffic=stored_traffic(dom),
                    algorithmic_bytes=kern[dom]["bytes"])

    result = dict(
        metric=METRIC, value=round(value, 1), unit="GB/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=round(ms_per_step, 4), higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype="fp32", data="synthetic",
        config=dict(workload=f"fused layer ops at T={T}: residual-add+RMSNorm->FP8 per-token "
                             f"(H=4096), SiLU-and-Mul->FP8 group-128 (I=14336), neox RoPE->paged "
                             f"KV write (32/8 heads x 128, cache 4096x16x8x128), MLA dual RMSNorm "
                             f"(1536 FP8 group-128 / 512 bf16)",
                    T=T, io="bf16 in; e4m3fn codes + fp32 scales / bf16 out; fp32 arithmetic",
                    step_bytes=step_bytes),
        settle=dict(ms=args.settle_ms, steps=settled,
                    from_idle_ms_per_step=round(idle_wall / args.steps * 1e3, 4),
                    from_idle_value=round(step_bytes / (idle_wall / args.steps) / 1e9, 1)),
        kernels=kern, roofline=roofline, env=environment(),
        target=dict(frac_of_peak=TARGET_FRAC,
                    met=[n for n in KERNELS if kern[n]["meets_target"]],
                    missed=[n for n in KERNELS if not kern[n]["meets_target"]],
                    timing="HIP events around each launch of the timed steps (mean)"),
    )
    ceiling = copy_ceiling()
    for n in KERNELS:
        kern[n]["frac_of_copy"] = round(kern[n]["gbps"] / ceiling["gbps"], 4)
    result["copy_ceiling"] = ceiling
    # The same kernels timed the way the copy ceiling is: alone, back to back,
    # one event pair around all launches (no event between two kernels).
    b2b = back_to_back(T)
    for n in KERNELS:
        ms = b2b[n]
        gbps = algo_bytes(n, T) / (ms * 1e-3) / 1e9
        kern[n]["back_to_back"] = dict(us=round(ms * 1e3, 2), gbps=round(gbps, 1),
                                       frac_of_peak=round(gbps / PEAK_HBM_GBPS, 4),
                                       frac_of_copy=round(gbps / ceiling["gbps"], 4),
                                       meets_target=gbps / PEAK_HBM_GBPS >= TARGET_FRAC)
    result["target"]["met_back_to_back"] = [n for n in KERNELS
                                            if kern[n]["back_to_back"]["meets_target"]]
    result["target"]["missed_back_to_back"] = [n for n in KERNELS
                                               if not kern[n]["back_to_back"]["meets_target"]]
    if args.next_rows:
        result["next_rows"] = {r["kernel"]: {k: v for k, v in r.items() if k != "kernel"}
                               for r in sweep([T], kernels=NEXT_KERNELS)}
    if args.modes:
        result["modes"] = {r["kernel"]: {k: v for k, v in r.items() if k != "kernel"}
                           for r in sweep([T], kernels=MODE_KERNELS)}
    if args.fusion:
        result["fusion"] = fusion_report(kern, T, dual_two_launch(sorted({64, 1024, T})))
    if args.decode:
        try:
            result["decode"] = decode_steps([int(t) for t in args.decode.split(",") if t])
        except Exception as e:  # a measurement beside the step: record it, keep the line
            result["decode"] = dict(error=f"{type(e).__name__}: {e}")
            log(f"decode timing failed: {e}")
    if args.sweep:
        result["sweep"] = sweep([int(t) for t in args.sweep.split(",") if t],
                                kernels=_sweep_kernels(args))
        hip = HipEvents()
        floor_ms, _ = copy_yardstick(8192, 30, hip, torch.cuda.current_stream().cuda_stream,
                                     _blocker_cycles())
        result["launch_floor_us"] = round(floor_ms * 1e3, 2)
        log(f"launch floor (one-workgroup copy, timed as the sweep): {floor_ms * 1e3:.2f} us")
    if args.cpu_sample > 0:
        result["cpu_baseline"] = cpu_baseline(args.cpu_sample, min(1024, args.cpu_sample))
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
