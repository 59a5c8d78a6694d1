"""Mutation check of the oracle's pins (test infrastructure, CPU only).

Each mutant plants one plausible mistake in a copy of oracle/rra_oracle.c (a
dropped term, a wrong sign, index, operand or stride), rebuilds that copy with
gcc in a temporary directory and runs the oracle's pins (tests/test_oracle_*.py,
`-m "not gpu"`) against it.  A mutant is caught when a pin fails.  The
repository itself is never modified.

    python oracle/mutation_check.py            # all mutants, 4 at a time
    python oracle/mutation_check.py --only 3 7 # some of them
"""
from __future__ import annotations

import argparse
import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, text in rra_oracle.c, replacement).  The first occurrence of the text
# is replaced: where a text occurs more than once, the first is the fused op's
# (the unfused compositions and the other ops follow it in the file).  The
# entries of BOTH_MUTANTS replace every occurrence, so that the fused and the
# unfused function carry the same mistake and the fused == unfused pins cannot
# see it; an entry whose text and replacement are tuples plants each pair.
MUTANTS = [
    # residual add + RMSNorm + FP8 quant
    ("eps outside the root", "1.0 / sqrt(ss / (double)H + (double)eps)",
     "1.0 / (sqrt(ss / (double)H) + (double)eps)"),
    ("weight taken as 1 + w", "y[j] = z[j] * rho * elem_decode(w[j], dtype);",
     "y[j] = z[j] * rho * (1.0 + elem_decode(w[j], dtype));"),
    ("mean over H - 1", "sqrt(ss / (double)H + (double)eps)",
     "sqrt(ss / (double)(H - 1) + (double)eps)"),
    ("scale amax / 447", "amax / 448.0", "amax / 447.0"),
    ("quantize by the reciprocal", "orc_e4m3fn_encode(y / (double)s)",
     "orc_e4m3fn_encode(y * (1.0 / (double)s))"),
    ("group amax misses a column",
     "for (int64_t j = g0; j < g0 + group_size; ++j) amax",
     "for (int64_t j = g0; j < g0 + group_size - 1; ++j) amax"),
    ("signed amax (per token)",
     "for (int64_t j = 0; j < H; ++j) amax = fmax(amax, fabs(y[j]));",
     "for (int64_t j = 0; j < H; ++j) amax = fmax(amax, y[j]);"),
    ("group scale stride",
     "if (mode == ORC_Q_PER_GROUP) return scales + t * (H / group_size);",
     "if (mode == ORC_Q_PER_GROUP) return scales + t * (H / group_size - 1);"),
    ("norm input is the unrounded sum",
     "        const uint16_t zb = orc_bf16_encode(xv + orc_bf16_decode(residual[t * res_stride + j]));\n"
     "        residual[t * res_stride + j] = zb;\n"
     "        z[j] = orc_bf16_decode(zb);",
     "        const double ex = xv + orc_bf16_decode(residual[t * res_stride + j]);\n"
     "        const uint16_t zb = orc_bf16_encode(ex);\n"
     "        residual[t * res_stride + j] = zb;\n"
     "        z[j] = ex;"),
    ("residual not written back",
     "        residual[t * res_stride + j] = zb;\n        z[j] = orc_bf16_decode(zb);",
     "        z[j] = orc_bf16_decode(zb);"),
    # SiLU-and-Mul + FP8 quant
    ("SiLU halves swapped",
     "a[j] = silu_mul(orc_bf16_decode(row[j]), orc_bf16_decode(row[I + j]));",
     "a[j] = silu_mul(orc_bf16_decode(row[I + j]), orc_bf16_decode(row[j]));"),
    ("sigmoid sign", "g / (1.0 + exp(-g)) * u", "g / (1.0 + exp(g)) * u"),
    # RoPE + paged KV write
    ("RoPE sin sign", "out[a] = elem_encode(x[a] * c[i] - x[b] * s[i], dtype);",
     "out[a] = elem_encode(x[a] * c[i] + x[b] * s[i], dtype);"),
    ("RoPE frequency exponent", "pow(theta, -2.0 * (double)i / (double)rot_dim)",
     "pow(theta, -1.0 * (double)i / (double)rot_dim)"),
    ("RoPE pairing swapped",
     "const int a = is_neox ? i : 2 * i;\n    const int b = is_neox ? i + half : 2 * i + 1;",
     "const int a = is_neox ? 2 * i : i;\n    const int b = is_neox ? 2 * i + 1 : i + half;"),
    ("RoPE position off by one", "rope_angles(positions[t], theta, rot_dim, c, s);",
     "rope_angles(positions[t] + 1, theta, rot_dim, c, s);"),
    ("slot block and offset swapped",
     "const int64_t blk = slot / block_size, off = slot % block_size;",
     "const int64_t blk = slot % block_size, off = slot / block_size;"),
    ("k copied as v",
     "memcpy(cache_head(value_cache, slot, block_size, Hkv, D, h),\n               v + t * v_stride",
     "memcpy(cache_head(value_cache, slot, block_size, Hkv, D, h),\n               k + t * k_stride"),
    # MLA dual RMSNorm
    ("MLA: kv uses the q epsilon", "norm_emit_row(kv + t * kv_stride, kv_w, eps_kv,",
     "norm_emit_row(kv + t * kv_stride, kv_w, eps_q,"),
    ("MLA: kv uses the q weight", "norm_emit_row(kv + t * kv_stride, kv_w, eps_kv,",
     "norm_emit_row(kv + t * kv_stride, q_w, eps_kv,"),
    ("MLA: q uses the kv epsilon", "norm_emit_row(q + t * q_stride, q_w, eps_q, Hq,",
     "norm_emit_row(q + t * q_stride, q_w, eps_kv, Hq,"),
    # QK norm + RoPE (+ KV write)
    ("QK norm: q heads use the k weight",
     "norm_rope_head(row + (int64_t)h * D, q_weight,",
     "norm_rope_head(row + (int64_t)h * D, k_weight,"),
    ("QK norm: k heads use the q weight",
     "norm_rope_head(k + (int64_t)h * D, k_weight,",
     "norm_rope_head(k + (int64_t)h * D, q_weight,"),
    ("QK norm: cache gets the raw k",
     "memcpy(cache_head(key_cache, slot, block_size, Hkv, D, h), kr,",
     "memcpy(cache_head(key_cache, slot, block_size, Hkv, D, h), k + (int64_t)h * D,"),
    ("QK norm: write_k ignored", "if (write_k) memcpy(k + (int64_t)h * D, kr,",
     "if (0) memcpy(k + (int64_t)h * D, kr,"),
    ("QK norm: v cache from the k head",
     "memcpy(cache_head(value_cache, slot, block_size, Hkv, D, h), v + (int64_t)h * D,",
     "memcpy(cache_head(value_cache, slot, block_size, Hkv, D, h), k + (int64_t)h * D,"),
    # residual add + RMSNorm + padding
    ("padding: tail not zero", "for (int64_t j = H; j < H_pad; ++j) o[j] = 0;",
     "for (int64_t j = H; j < H_pad; ++j) o[j] = 0x3F80;"),
    ("padding: norm input is the unrounded sum",
     "        rr[j] = elem_encode(z[j] + elem_decode(rr[j], dtype), dtype);\n"
     "        z[j] = elem_decode(rr[j], dtype);",
     "        const double ex = z[j] + elem_decode(rr[j], dtype);\n"
     "        rr[j] = elem_encode(ex, dtype);\n"
     "        z[j] = ex;"),
    # MLA k_pe RoPE + [kv_c | k_pe] cache write
    ("MLA RoPE: q head stride", "uint16_t* qh = q_pe + t * q_stride + (int64_t)h * q_head_stride;",
     "uint16_t* qh = q_pe + t * q_stride + (int64_t)h * rope_dim;"),
    ("MLA RoPE: kv_c copied from one element on",
     "memcpy(dst, kv_c + t * kv_c_stride, (size_t)kv_lora * sizeof(uint16_t));",
     "memcpy(dst, kv_c + t * kv_c_stride + 1, (size_t)kv_lora * sizeof(uint16_t));"),
    ("MLA RoPE: k_pe pairing flipped",
     "rotate_head(k_pe + t * k_pe_stride, dst + kv_lora, c, s, rope_dim, rope_dim, is_neox,",
     "rotate_head(k_pe + t * k_pe_stride, dst + kv_lora, c, s, rope_dim, rope_dim, !is_neox,"),
    # codecs and element types
    ("E4M3 ties away from zero", "    k = (lo % 2 == 0) ? lo : hi;", "    k = hi;"),
    ("E4M3 overflows to NaN above 464", "  if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);",
     "  if (a > 464.0) return (uint8_t)(sign | 0x7Fu);\n"
     "  if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);"),
    ("E4M3 subnormal step 2^-10", "    mag = ldexp((double)m, -9);",
     "    mag = ldexp((double)m, -10);"),
    ("bf16 rounding truncates", "  const double n = nearbyint(a / quantum);",
     "  const double n = floor(a / quantum);"),
    ("fp16 rounding truncates",
     "  const double r = nearbyint(a / ldexp(1.0, E - 10)) * ldexp(1.0, E - 10);",
     "  const double r = floor(a / ldexp(1.0, E - 10)) * ldexp(1.0, E - 10);"),
    ("fp16 subnormal binade clamped at -15", "  if (E < -14) E = -14;",
     "  if (E < -15) E = -15;"),
    ("fp16 exponent bias 14", "    mag = ldexp(1.0 + (double)f / 1024.0, e - 15);",
     "    mag = ldexp(1.0 + (double)f / 1024.0, e - 14);"),
    ("fp16 elements read as bf16",
     "  return dtype == ORC_DT_F16 ? orc_f16_decode(h) : orc_bf16_decode(h);",
     "  return orc_bf16_decode(h);"),
    # quantization and RoPE, further slips
    ("quantize multiplies by the scale", "orc_e4m3fn_encode(y / (double)s)",
     "orc_e4m3fn_encode(y * (double)s)"),
    ("RoPE tail zeroed past rot_dim", "  for (int d = rot_dim; d < D; ++d) out[d] = keep[d];",
     "  for (int d = rot_dim; d < D; ++d) out[d] = 0;"),
]


BOTH_MUTANTS = [
    ("MLA, fused and unfused: kv uses the q epsilon",
     "norm_emit_row(kv + t * kv_stride, kv_w, eps_kv,",
     "norm_emit_row(kv + t * kv_stride, kv_w, eps_q,"),
    ("MLA, fused and unfused: kv uses the q weight",
     "norm_emit_row(kv + t * kv_stride, kv_w, eps_kv,",
     "norm_emit_row(kv + t * kv_stride, q_w, eps_kv,"),
    ("residual-add norm, fused and unfused: norm input is the unrounded sum",
     ("        const uint16_t zb = orc_bf16_encode(xv + orc_bf16_decode(residual[t * res_stride + j]));\n"
      "        residual[t * res_stride + j] = zb;\n"
      "        z[j] = orc_bf16_decode(zb);",
      "        const uint16_t zb = orc_bf16_encode(v + orc_bf16_decode(residual[t * res_stride + j]));\n"
      "        residual[t * res_stride + j] = zb;\n"
      "        v = orc_bf16_decode(zb);"),
     ("        const double ex = xv + orc_bf16_decode(residual[t * res_stride + j]);\n"
      "        residual[t * res_stride + j] = orc_bf16_encode(ex);\n"
      "        z[j] = ex;",
      "        const double ex = v + orc_bf16_decode(residual[t * res_stride + j]);\n"
      "        residual[t * res_stride + j] = orc_bf16_encode(ex);\n"
      "        v = ex;")),
    # The unfused form normalizes a quantized q through the residual-add norm's
    # function, so the mistake is planted at that call too.
    ("MLA, fused and unfused: q uses the kv epsilon",
     ("norm_emit_row(q + t * q_stride, q_w, eps_q, Hq,",
      "orc_fused_add_rmsnorm_quant(q, q_stride, NULL, 0, q_w, eps_q, q_quant_mode"),
     ("norm_emit_row(q + t * q_stride, q_w, eps_kv, Hq,",
      "orc_fused_add_rmsnorm_quant(q, q_stride, NULL, 0, q_w, eps_kv, q_quant_mode")),
]
ALL = [(n, o, r, False) for n, o, r in MUTANTS] + [(n, o, r, True) for n, o, r in BOTH_MUTANTS]


# What the oracle's tests need: the oracle itself, the tests, the seeded input
# generators and the pytest configuration.
COPIED = ("oracle", "tests", "workloads.py", "pytest.ini")


def _copy_tree(dst: str) -> None:
    os.makedirs(dst)
    skip = shutil.ignore_patterns("__pycache__", "*.so", ".pytest_cache")
    for name in COPIED:
        src = os.path.join(ROOT, name)
        if os.path.isdir(src):
            shutil.copytree(src, os.path.join(dst, name), ignore=skip)
        else:
            shutil.copy2(src, os.path.join(dst, name))


def run_one(i: int) -> tuple:
    name, old, new, every = ALL[i]
    with tempfile.TemporaryDirectory(prefix="orc_mut_") as tmp:
        d = os.path.join(tmp, "repo")
        _copy_tree(d)
        src = os.path.join(d, "oracle", "rra_oracle.c")
        text = open(src, encoding="utf-8").read()
        pairs = zip(old, new) if isinstance(old, tuple) else [(old, new)]
        for o, r in pairs:
            if o not in text:
                return i, name, "text not found (not applied)"
            text = text.replace(o, r, -1 if every else 1)
        open(src, "w", encoding="utf-8").write(text)
        r = subprocess.run([sys.executable, "-c", "import oracle; oracle.build()"], cwd=d,
                           capture_output=True, text=True)
        if r.returncode:
            return i, name, "build failed: " + r.stderr[-200:]
        tests = sorted(os.path.join("tests", f) for f in os.listdir(os.path.join(d, "tests"))
                       if f.startswith("test_oracle_") and f.endswith(".py"))
        env = dict(os.environ, OMP_NUM_THREADS="2")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p",
                            "no:cacheprovider", *tests], cwd=d, capture_output=True, text=True,
                           timeout=1800, env=env)
        if r.returncode == 0:
            return i, name, "NOT CAUGHT"
        failed = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED")]
        pin = failed[0].split(" ")[1] if failed else "an error in the run"
        return i, name, "caught by " + pin


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--only", type=int, nargs="*")
    ap.add_argument("--workers", type=int, default=4)
    a = ap.parse_args()
    which = a.only if a.only else range(len(ALL))
    results = []
    with concurrent.futures.ThreadPoolExecutor(a.workers) as ex:
        for i, name, verdict in ex.map(run_one, which):
            print(f"{i:2d} {name}: {verdict}", flush=True)
            results.append(verdict)
    caught = sum(v.startswith("caught") for v in results)
    print(f"{caught} of {len(results)} mutants caught", flush=True)
    return 0 if caught == len(results) else 1


if __name__ == "__main__":
    sys.exit(main())
