"""rocprofv3 output summaries for profiles/ (kernel-trace statistics and HBM byte counters).

Usage:
  python -m block_sparse_attention_quest_amd.profiling stats <kernel_stats.csv> <out.md> "<command>"
        [--trace <kernel_trace.csv>] [--bench-log <bench.py output of the same run>]
  python -m block_sparse_attention_quest_amd.profiling hbm <fetch counter_collection.csv>
        <write counter_collection.csv> <out.md> --copy-mib N "<fetch command>" "<write command>"
  python -m block_sparse_attention_quest_amd.profiling sq <counter_collection.csv>... <out.md>
        --bench-log <bench.py output of the first run> "<command>"...

`stats` turns rocprofv3 --kernel-trace --stats output into a short table; with the kernel trace and the
bench.py output of the same run it also records the mean duration of the speculative-attention launches
bench.py timed alone (keyed by the attention source hash, for bench.py to report beside its own figure).  `hbm` takes FETCH_SIZE and
WRITE_SIZE (KiB per dispatch) of every speculative-attention launch, scales each counter by what it reads
for a plain device copy of known size (the copy probe bench.py runs with --copy-probe-mib: the copy
kernel with the largest WRITE_SIZE, matched by dispatch id in the FETCH_SIZE run), and
records the attention source hash so that bench.py ignores the numbers once the kernel changes.  `sq`
summarises SQ counter runs (wave cycles spent waiting and issuing, vector-memory reads and MFMA per wave,
vector-memory latency) per kernel role.
"""
from __future__ import annotations

import csv
import hashlib
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
SPEC_KERNEL = "attn_spec_bf16"


def kernel_source_hash() -> str:
    """sha256 (first 16 hex digits) of the attention kernel source (device code and kernel file)."""
    h = hashlib.sha256()
    for name in ("attn_core.hpp", "attn.hip"):
        with open(os.path.join(PKG, "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    n = name
    for pre in ("void ", "prr::(anonymous namespace)::"):
        n = n.replace(pre, "")
    return n.split("(")[0][:70]


def _get(row: dict, *keys, default=""):
    for k in keys:
        if k in row:
            return row[k]
    return default


def stats_table(path: str, top: int = 16) -> str:
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(_get(r, "TotalDurationNs", default=0)))
    out = ["| kernel | calls | avg us | min us | max us | total % |", "|---|---|---|---|---|---|"]
    for r in rows[:top]:
        out.append("| `{}` | {} | {:.2f} | {:.2f} | {:.2f} | {:.1f} |".format(
            _short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(_get(r, "Percentage", default=0))))
    return "\n".join(out)


def trace_averages(path: str, names=("spec", "repair", "select_spec", "layer_step")) -> str:
    """Average and median duration of each named kernel per stream over its launches that did work:
    launches shorter than a fifth of the kernel's longest (calls over empty sets) are left out; the
    warm-up steps' launches, which run slower, stay in (the median is the figure to compare with a
    timed run).  The
    stream that also runs the cache-flush reductions is the one bench.py times kernels alone on; the
    other carries the overlapped layer step's speculative pass."""
    rows = list(csv.DictReader(open(path)))
    flush_streams = {r["Stream_Id"] for r in rows if "reduce_kernel" in r["Kernel_Name"]}
    out = ["| kernel (role) | stream | launches with work | avg us | median us | min us | max us |",
           "|---|---|---|---|---|---|---|"]
    for nm in names:
        sel = [r for r in rows if kernel_role(r["Kernel_Name"]) == nm]
        if not sel:
            continue
        dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        top = max(dur(r) for r in sel)
        for sid in sorted({r["Stream_Id"] for r in sel}):
            ds = [dur(r) for r in sel if r["Stream_Id"] == sid and dur(r) >= 0.2 * top]
            if not ds:
                continue
            kind = "flush stream (isolated launches + critical path)" if sid in flush_streams else "side stream"
            out.append(f"| {nm} | {sid}: {kind} | {len(ds)} | {statistics.mean(ds):.2f} | "
                       f"{statistics.median(ds):.2f} | {min(ds):.2f} | {max(ds):.2f} |")
    return "\n".join(out)


def spec_timed_launches(path: str, skip: int, kernel: str = SPEC_KERNEL) -> list:
    """Durations (us) of the speculative-attention launches bench.py times alone: the launches on the
    stream that also runs the cache-flush reductions (the side stream carries the three-stream
    schedule's launches), after the first `skip` (the warm-up steps')."""
    rows = list(csv.DictReader(open(path)))
    flush_streams = {r["Stream_Id"] for r in rows if "reduce_kernel" in r["Kernel_Name"]}
    sel = [r for r in rows if kernel in r["Kernel_Name"] and r["Stream_Id"] in flush_streams]
    sel.sort(key=lambda r: int(r["Start_Timestamp"]))
    return [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in sel[skip:]]


def bench_line(log_path: str) -> dict:
    import json

    line = [ln for ln in open(log_path) if ln.startswith('{"metric"')][-1]
    return json.loads(line)


def bench_in_run(d: dict, spec_rocprof: list) -> list:
    """bench.py's own figures from the JSON line of the profiled run beside rocprofv3's, for the
    cross-check of the two clocks on the same launches."""
    rows = ["bench.py's own figures in the same (profiled) run: the GPU time of each call's kernels from HIP "
            "events bound to the launches (prr_time_next_kernel), over the timed steps:", "",
            "| kernel | bench.py us (median) |", "|---|---|"]
    for key, name in (("us_spec_attn_median", "attn_spec_bf16"), ("us_repair_median", "attn_repair_bf16"),
                      ("us_select_spec_median", "select_spec_kernel")):
        if d.get(key) is not None:
            rows.append(f"| `{name}` | {d[key]:.2f} |")
    rf = d.get("roofline", {})
    if rf.get("avg_launch_us") is not None and spec_rocprof:
        r = statistics.mean(spec_rocprof)
        rows += ["", f"Speculative pass, mean over the {len(spec_rocprof)} timed launches: bench.py "
                 f"{rf['avg_launch_us']:.2f} us, rocprofv3 {r:.2f} us "
                 f"({100.0 * (rf['avg_launch_us'] - r) / r:+.2f}%)."]
    return rows


def _per_dispatch(path: str, counter: str) -> dict:
    """{dispatch id: (kernel name, summed counter value)} for one counter."""
    out = {}
    for r in csv.DictReader(open(path)):
        if _get(r, "Counter_Name", "Counter-Name") != counter:
            continue
        did = int(_get(r, "Dispatch_Id", "Dispatch-Id"))
        name = _get(r, "Kernel_Name", "Kernel-Name")
        val = float(_get(r, "Counter_Value", "Counter-Value", default=0))
        prev = out.get(did, (name, 0.0))
        out[did] = (name, prev[1] + val)
    return out


def hbm_summary(fetch_csv: str, write_csv: str, copy_mib: int, kernel: str = None) -> dict:
    """HBM bytes per launch of `kernel` (default: the speculative-attention kernel) from FETCH_SIZE and
    WRITE_SIZE, each scaled by its reading for the probe copy of copy_mib MiB in the same run."""
    kernel = kernel or SPEC_KERNEL
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    # the probe copy: the copy kernel with the largest write, matched by dispatch id across the runs
    copies = [(v, d) for d, (n, v) in write.items() if "copyBuffer" in n]
    if not copies:
        raise SystemExit("no copy dispatch found in the WRITE_SIZE run")
    copy_write, copy_id = max(copies)
    copy_fetch = fetch[copy_id][1]
    known = copy_mib * 1024.0   # KiB read and written by the probe copy
    f_scale = known / copy_fetch
    w_scale = known / copy_write
    sel = [(d, f, write[d][1]) for d, (n, f) in sorted(fetch.items()) if kernel in n and d in write]
    if not sel:
        return None
    top = max(f for _, f, _ in sel)
    sel = [x for x in sel if x[1] >= 0.1 * top]   # launches over an empty set (warm-up) carry no K/V
    per_launch = [(f * f_scale + wv * w_scale) * 1024.0 for _, f, wv in sel]
    # the median: a few launches of a run work on other sets (the first decode step has P empty, so its
    # repair covers all of A and its speculative part is empty)
    return {"spec_dispatches": len(sel), "fetch_kib_mean": statistics.median(f for _, f, _ in sel),
            "write_kib_mean": statistics.median(wv for _, _, wv in sel), "copy_fetch_kib": copy_fetch,
            "copy_write_kib": copy_write, "fetch_scale": f_scale, "write_scale": w_scale,
            "hbm_bytes_per_launch": statistics.median(per_launch)}


def kernel_role(name: str):
    """The role of a kernel of the path, by its (demangled) name: the keys of bench.py's
    algorithmic_bytes_per_launch, plus the calibration, metadata and top-K stage kernels."""
    if "attn_spec_" in name:
        return "spec"
    if "attn_repair_" in name:
        return "repair"
    if "select_spec_kernel" in name:
        # template arguments <cache type, d, keys per thread, two-stage, mean, carried predictor, repair>
        targs = name[name.index("<") + 1:].split(">")[0].split(",") if "<" in name else []
        return "layer_step" if len(targs) >= 7 and targs[6].strip() == "true" else "select_spec"
    # calibration first: its per-row ranking kernel is also a top-K kernel
    for key, role in (("rows_topk_kernel", "calibration: rows' true top-K"), ("ema_chain_kernel", "calibration: EMA chain"),
                      ("replay_kernel", "calibration: replay"), ("score_kernel", "score"), ("score_parts_kernel", "score"),
                      ("topk_groups_kernel", "topk_groups"), ("topk_kernel", "topk"), ("predict", "predict"),
                      ("summary_kernel", "meta"), ("meta_kernel", "meta"), ("append", "append")):
        if key in name:
            return role
    return None


def roles_table(fetch_csv: str, write_csv: str, copy_mib: int, algo: dict = None) -> list:
    """Per role: dispatches that did work, median HBM bytes per launch (FETCH_SIZE and WRITE_SIZE scaled
    by the copy probe), and with bench.py's algorithmic bytes per launch the ratio of the two."""
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    copies = [(v, d) for d, (n, v) in write.items() if "copyBuffer" in n]
    if not copies:
        raise SystemExit("no copy dispatch found in the WRITE_SIZE run")
    copy_write, copy_id = max(copies)
    f_scale = copy_mib * 1024.0 / fetch[copy_id][1]
    w_scale = copy_mib * 1024.0 / copy_write
    by_role = {}
    for d, (n, f) in fetch.items():
        role = kernel_role(n)
        if role and d in write:
            by_role.setdefault(role, []).append((f * f_scale + write[d][1] * w_scale) * 1024.0)
    out = ["| kernel (role) | dispatches | HBM bytes per launch, median | algorithmic bytes per launch | "
           "HBM / algorithmic |", "|---|---|---|---|---|"]
    for role in ("spec", "repair", "select_spec", "layer_step", "score", "topk", "topk_groups", "predict",
                 "calibration: rows' true top-K", "calibration: EMA chain", "calibration: replay", "meta", "append"):
        xs = by_role.get(role)
        if not xs:
            continue
        top = max(xs)
        xs = [x for x in xs if x >= 0.1 * top]   # launches over empty sets (warm-up, first step) left out
        med = statistics.median(xs)
        a = (algo or {}).get(role)
        ratio = f"{med / a:.3f}" if a else "-"
        out.append(f"| {role} | {len(xs)} | {med:.0f} | {a:.0f} | {ratio} |" if a else
                   f"| {role} | {len(xs)} | {med:.0f} | - | - |")
    return out


def _per_dispatch_all(path: str) -> dict:
    """{dispatch id: (kernel name, {counter: value summed over instances})} for every counter of a run."""
    out = {}
    for r in csv.DictReader(open(path)):
        did = int(_get(r, "Dispatch_Id", "Dispatch-Id"))
        name = _get(r, "Kernel_Name", "Kernel-Name")
        c = _get(r, "Counter_Name", "Counter-Name")
        val = float(_get(r, "Counter_Value", "Counter-Value", default=0))
        entry = out.setdefault(did, (name, {}))
        entry[1][c] = entry[1].get(c, 0.0) + val
    return out


def sq_table(paths: list) -> list:
    """Per role, medians over the launches that did work (SQ_WAVE_CYCLES at least a tenth of the role's
    largest) of: the share of the waves' cycles spent waiting (SQ_WAIT_ANY / SQ_WAVE_CYCLES, both in
    quad-cycles), the share spent issuing (SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES), vector-memory reads and
    MFMA instructions per wave, and the average vector-memory latency in cycles (VmemLatency, from its
    own run)."""
    per_role = {}
    for path in paths:
        for did, (name, cs) in _per_dispatch_all(path).items():
            role = kernel_role(name)
            if role is not None:
                per_role.setdefault(role, {}).setdefault(path, []).append(cs)
    rows = ["| kernel (role) | launches | waiting, % of wave cycles | issuing, % of wave cycles | vector-memory reads per wave | MFMA per wave | vector-memory latency, cycles |",
            "|---|---|---|---|---|---|---|"]
    order = ["spec", "repair", "select_spec", "layer_step", "score", "topk", "topk_groups", "predict"]
    for role in [r for r in order if r in per_role] + [r for r in per_role if r not in order]:
        vals = {}
        n = 0
        for path, lst in per_role[role].items():
            if any("SQ_WAVE_CYCLES" in cs for cs in lst):
                top = max(cs.get("SQ_WAVE_CYCLES", 0.0) for cs in lst)
                lst = [cs for cs in lst if cs.get("SQ_WAVE_CYCLES", 0.0) >= 0.1 * top]
                n = max(n, len(lst))
            for cs in lst:
                for k, v in cs.items():
                    vals.setdefault(k, []).append(v)
        med = {k: statistics.median(v) for k, v in vals.items()}
        def share(a, b):
            return f"{100.0 * med[a] / med[b]:.1f}" if a in med and b in med and med[b] > 0 else "-"
        def per_wave(a):
            return f"{med[a] / med['SQ_WAVES']:.1f}" if a in med and med.get("SQ_WAVES", 0) > 0 else "-"
        lat = f"{med['VmemLatency']:.0f}" if "VmemLatency" in med else "-"
        rows.append(f"| {role} | {n} | {share('SQ_WAIT_ANY', 'SQ_WAVE_CYCLES')} | {share('SQ_ACTIVE_INST_ANY', 'SQ_WAVE_CYCLES')} "
                    f"| {per_wave('SQ_INSTS_VMEM_RD')} | {per_wave('SQ_INSTS_MFMA')} | {lat} |")
    return rows


def main(argv):
    if argv and argv[0] == "stats":
        _, src, out, cmd = argv[:4]
        text = ["# Kernel statistics (rocprofv3 --kernel-trace --stats)", "", "Command:", "", "```", cmd, "```",
                "", stats_table(src), ""]
        d = bench_line(argv[argv.index("--bench-log") + 1]) if "--bench-log" in argv else None
        spec = []
        if "--trace" in argv:
            trace = argv[argv.index("--trace") + 1]
            text += ["Attention launches over non-empty sets (from the kernel trace of the same run):", "",
                     trace_averages(trace), ""]
            if d is not None:
                spec = spec_timed_launches(trace, int(d.get("warmup", 0)))
                spec = spec[-int(d["steps"]):]
        if spec:
            text += [f"- kernel: `{SPEC_KERNEL}<128>`",
                     f"- kernel_source_sha256: `{kernel_source_hash()}`",
                     f"- attn_spec_timed_launches: {len(spec)}",
                     f"- attn_spec_avg_us: {statistics.mean(spec):.3f}",
                     f"- attn_spec_median_us: {statistics.median(spec):.3f}", ""]
        if d is not None:
            text += bench_in_run(d, spec) + [""]
        open(out, "w").write("\n".join(text))
        print("\n".join(text))
    elif argv and argv[0] == "hbm":
        fetch_csv, write_csv, out = argv[1:4]
        i = argv.index("--copy-mib")
        copy_mib = int(argv[i + 1])
        cmds = [a for k, a in enumerate(argv[4:], start=4) if k not in (i, i + 1)]
        d = None
        if "--bench-log" in argv:
            j = argv.index("--bench-log")
            d = bench_line(argv[j + 1])
            cmds = [a for a in cmds if a not in (argv[j], argv[j + 1])]
        s = hbm_summary(fetch_csv, write_csv, copy_mib)
        title = "the path's kernels" if s is None else "the speculative-attention kernel and the path's kernels"
        workload = f" ({d['config']['workload']})" if d else ""
        lines = [f"# HBM traffic of {title}{workload} (rocprofv3 --pmc)", "",
                 "FETCH_SIZE and WRITE_SIZE are KiB per dispatch; each is scaled by what it reads for a "
                 f"{copy_mib} MiB device copy (known bytes read and written) in the same run.", "",
                 "Commands:", "", "```", *cmds, "```", ""]
        if s is not None:
            lines += [f"- kernel: `{SPEC_KERNEL}<128>`",
                      f"- kernel_source_sha256: `{kernel_source_hash()}`",
                      f"- spec_dispatches: {s['spec_dispatches']}",
                      f"- fetch_kib_per_dispatch_median: {s['fetch_kib_mean']:.1f}",
                      f"- write_kib_per_dispatch_median: {s['write_kib_mean']:.1f}",
                      f"- copy_fetch_kib: {s['copy_fetch_kib']:.1f}",
                      f"- copy_write_kib: {s['copy_write_kib']:.1f}",
                      f"- fetch_scale: {s['fetch_scale']:.4f}",
                      f"- write_scale: {s['write_scale']:.4f}",
                      f"- hbm_bytes_per_launch: {s['hbm_bytes_per_launch']:.0f}", ""]
        lines += ["Every kernel of the path in the same runs (same scaling; launches that did work; algorithmic "
                  "bytes from bench.py's algorithmic_bytes_per_launch of the run):", ""]
        lines += roles_table(fetch_csv, write_csv, copy_mib, d.get("algorithmic_bytes_per_launch") if d else None)
        lines.append("")
        open(out, "w").write("\n".join(lines))
        print("\n".join(lines))
    elif argv and argv[0] == "sq":
        # sq <counters.csv>... <out.md> --bench-log <log> <commands>...
        j = argv.index("--bench-log")
        d = bench_line(argv[j + 1])
        head = argv[1:j]
        csvs, out = head[:-1], head[-1]
        cmds = argv[j + 2:]
        lines = [f"# Where the waves' time goes ({d['config']['workload']}; rocprofv3 --pmc, SQ counters)", "",
                 "Per kernel role, medians over the launches that did work; the counters are summed over the "
                 "GPU per dispatch. Waiting and issuing are shares of the waves' cycles (SQ_WAIT_ANY and "
                 "SQ_ACTIVE_INST_ANY over SQ_WAVE_CYCLES); the latency is VmemLatency (in-flight vector-memory "
                 "instructions accumulated over their count).", "",
                 f"- attention kernel_source_sha256: `{kernel_source_hash()}`", "",
                 "Commands:", "", "```", *cmds, "```", ""]
        lines += sq_table(csvs)
        lines.append("")
        open(out, "w").write("\n".join(lines))
        print("\n".join(lines))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
