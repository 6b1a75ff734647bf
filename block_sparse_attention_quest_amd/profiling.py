"""rocprofv3 output summaries for profiles/ (kernel-trace statistics and HBM byte counters).

Usage:
  python -m block_sparse_attention_quest_amd.profiling stats <kernel_stats.csv> <out.md> "<command>"
  python -m block_sparse_attention_quest_amd.profiling hbm <fetch_counter_collection.csv>
        <write_counter_collection.csv> <out.md> "<commands>" [--copy-mib N]

`stats` turns rocprofv3 --kernel-trace --stats output into a short table.  `hbm` averages FETCH_SIZE and
WRITE_SIZE (KiB per dispatch) of the speculative-attention launches, scales them by what the same
counters read for a plain device copy of known size (the copy probe bench.py runs with
--copy-probe-mib), and records the attention source hash so stale numbers are ignored.
"""
from __future__ import annotations

import csv
import hashlib
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))


def kernel_source_hash() -> str:
    """sha256 (first 16 hex digits) of the attention kernel source."""
    with open(os.path.join(PKG, "csrc", "attn.hip"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _short(name: str) -> str:
    n = name.split("(")[0]
    for pre in ("void ", "prr::(anonymous namespace)::"):
        n = n.replace(pre, "")
    return n[:70]


def stats_table(path: str, top: int = 14) -> str:
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r.get("TotalDurationNs", 0)))
    out = ["| kernel | calls | avg us | min us | max us | total % |", "|---|---|---|---|---|---|"]
    for r in rows[:top]:
        out.append("| `{}` | {} | {:.2f} | {:.2f} | {:.2f} | {:.1f} |".format(
            _short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r.get("Percentage", 0))))
    return "\n".join(out)


def _counter_rows(path: str, counter: str):
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name", r.get("Counter-Name", "")) == counter:
            yield r


def _per_dispatch(path: str, counter: str, match) -> list:
    vals = {}
    for r in _counter_rows(path, counter):
        name = r.get("Kernel_Name", r.get("Kernel-Name", ""))
        if match(name):
            key = r.get("Dispatch_Id", r.get("Dispatch-Id", len(vals)))
            vals[key] = vals.get(key, 0.0) + float(r.get("Counter_Value", r.get("Counter-Value", 0)))
    return list(vals.values())


def hbm_summary(fetch_csv: str, write_csv: str, copy_mib: int, spec_calls_expected=None) -> dict:
    is_attn = lambda n: "attn_kernel" in n
    is_copy = lambda n: ("copy" in n.lower() or "elementwise" in n.lower()) and "attn" not in n
    f_attn = _per_dispatch(fetch_csv, "FETCH_SIZE", is_attn)
    w_attn = _per_dispatch(write_csv, "WRITE_SIZE", is_attn)
    f_copy = _per_dispatch(fetch_csv, "FETCH_SIZE", is_copy)
    w_copy = _per_dispatch(write_csv, "WRITE_SIZE", is_copy)
    known = copy_mib * 1024.0   # KiB read and written by the probe copy
    f_scale = known / max(f_copy) if f_copy and max(f_copy) > 0 else 1.0
    w_scale = known / max(w_copy) if w_copy and max(w_copy) > 0 else 1.0
    return {"attn_dispatches": len(f_attn), "fetch_kib_per_dispatch": f_attn, "write_kib_per_dispatch": w_attn,
            "copy_fetch_kib": max(f_copy) if f_copy else None, "copy_write_kib": max(w_copy) if w_copy else None,
            "fetch_scale": f_scale, "write_scale": w_scale}


def main(argv):
    if argv[0] == "stats":
        _, src, out, cmd = argv[:4]
        text = ["# Kernel statistics", "", "Command:", "", "```", cmd, "```", "", stats_table(src), ""]
        open(out, "w").write("\n".join(text))
    elif argv[0] == "hbm":
        fetch_csv, write_csv, out, cmd = argv[1:5]
        copy_mib = int(argv[argv.index("--copy-mib") + 1]) if "--copy-mib" in argv else 0
        s = hbm_summary(fetch_csv, write_csv, copy_mib)
        print(s)
        raise SystemExit("hbm summary printed; write the profile by hand from these numbers")
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
