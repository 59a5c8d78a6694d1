"""Summarize the parity figures that the GPU tests log (RRA_PARITY_LOG=path.jsonl)
into a markdown table: for every comparison, how many FP8 codes were compared
and how many differ from the oracle's (all by one code at most, or the test
fails), and the fraction of scales and bf16/fp16 outputs that are bit-identical
to the oracle's.

    RRA_PARITY_LOG=/tmp/parity.jsonl python -m pytest tests -m gpu -q
    python tests/parity_summary.py /tmp/parity.jsonl --out profiles/parity_every_row.md

Not a test module (pytest collects test_*.py only)."""
from __future__ import annotations

import argparse
import collections
import json


def load(path: str) -> list[dict]:
    with open(path, encoding="utf-8") as f:
        return [json.loads(line) for line in f if line.strip()]


def _module(test: str) -> str:
    return test.split("::", 1)[0].rsplit("/", 1)[-1] if test else "?"


def _headline(r: dict) -> bool:
    """The bench path and the workload cases at T = 8192 / 16384."""
    t = r.get("test", "")
    return "bench_path" in t or "T=8192" in r["what"] or "T=16384" in r["what"] or (
        "workload[8192]" in t or "workload[16384]" in t)


def summarize(recs: list[dict], command: str) -> str:
    mods = collections.OrderedDict()
    for r in recs:
        m = mods.setdefault(_module(r.get("test", "")), dict(codes=0, bad=0, mx=0, cases=set(),
                                                              exact=collections.Counter(),
                                                              n=collections.Counter()))
        m["cases"].add(r.get("test", ""))
        if r["kind"] == "codes":
            m["codes"] += r["codes"]
            m["bad"] += r["mismatches"]
            m["mx"] = max(m["mx"], r["max_ulp"])
        else:
            n = r.get("scales", r.get("values", 0))
            m["n"][r["kind"]] += n
            m["exact"][r["kind"]] += r["bit_exact_fraction"] * n
    out = ["# Parity against the oracle on every row (the GPU tests)", "",
           "Produced by (from the repository root):", "", "```", command, "```", "",
           "Every row (token) of every case is compared element by element with the oracle. "
           "Bars: FP8 codes at most one code apart on at most 1e-4 of them; scales and bf16 "
           "outputs within rtol 1e-2; fp16 within one fp16 unit; cache placement, copies and "
           "untouched slots bit-exact.", "",
           "## Per test module", "",
           "| module | cases | FP8 codes compared | differ | fraction | max ULP | scales "
           "bit-identical | bf16 bit-identical | fp16 bit-identical |",
           "|---|---|---|---|---|---|---|---|---|"]
    tot = [0, 0]
    for mod, m in mods.items():
        tot[0] += m["codes"]
        tot[1] += m["bad"]
        frac = lambda k: (f"{m['exact'][k] / m['n'][k]:.6f} of {m['n'][k]}" if m["n"][k]
                          else "-")
        out.append(f"| {mod} | {len(m['cases'])} | {m['codes']} | {m['bad']} | "
                   f"{m['bad'] / m['codes'] if m['codes'] else 0:.2e} | {m['mx']} | "
                   f"{frac('scales')} | {frac('bf16')} | {frac('f16')} |")
    out += ["", f"All modules: {tot[1]} of {tot[0]} codes differ from the oracle's "
                f"({tot[1] / tot[0] if tot[0] else 0:.2e}).", "",
            "## The headline sizes (T = 8192 and 16384, and the bench's own launch path)", "",
            "| test | comparison | values | differ / not bit-identical | fraction |",
            "|---|---|---|---|---|"]
    for r in recs:
        if not _headline(r):
            continue
        test = r.get("test", "").split("::", 1)[-1]
        if r["kind"] == "codes":
            out.append(f"| {test} | {r['what']} | {r['codes']} codes | {r['mismatches']} | "
                       f"{r['mismatches'] / r['codes'] if r['codes'] else 0:.2e} |")
        else:
            n = r.get("scales", r.get("values", 0))
            off = round((1.0 - r["bit_exact_fraction"]) * n)
            out.append(f"| {test} | {r['what']} | {n} {r['kind']} | {off} | "
                       f"{1.0 - r['bit_exact_fraction']:.2e} |")
    return "\n".join(out) + "\n"


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("log")
    ap.add_argument("--out")
    ap.add_argument("--command", help="the commands that produced the log, for the summary's "
                    "header (default: the usual two, with the log at {log})", default=(
        "RRA_PARITY_LOG={log} timeout -k 10 1000 python -u -m pytest tests "
        "-m gpu -x -q --timeout 300 --timeout-method thread\n"
        "python tests/parity_summary.py {log} --out profiles/parity_every_row.md"))
    a = ap.parse_args()
    text = summarize(load(a.log), a.command.replace("{log}", a.log))
    if a.out:
        with open(a.out, "w", encoding="utf-8") as f:
            f.write(text)
    else:
        print(text)


if __name__ == "__main__":
    main()
