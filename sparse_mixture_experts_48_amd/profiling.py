"""Summaries of rocprofv3 output for the layer's kernels.

Two kinds of summary, both short Markdown files:

* kernel trace (``rocprofv3 --kernel-trace --stats``): calls, mean and total
  duration of every kernel of a run;
* HBM traffic (two ``rocprofv3 --pmc`` runs, ``FETCH_SIZE`` then
  ``WRITE_SIZE``): bytes per launch of chosen kernels. Both counters are
  scaled by what they read for a plain device-to-device copy of known size
  taken in the same run (``bench.py --calibrate-copy MB``), so the figures are
  bytes, whatever unit the counters count in. The summary records the SHA-256
  of the source file of the kernels it measured; ``traffic_bytes`` returns
  nothing once that file has changed.

* counters (``rocprofv3 --pmc`` passes of SQ/GRBM counters): mean totals per
  launch of chosen kernels and the shares derived from them (MFMA busy, LDS
  bytes per clock, waiting wave-cycles).

Command line::

    python -m sparse_mixture_experts_48_amd.profiling trace STATS_CSV --command "..." > out.md
    python -m sparse_mixture_experts_48_amd.profiling counters A.csv B.csv --kernel gemm1=PATTERN \\
        --workload NAME --command "..." > out.md
    python -m sparse_mixture_experts_48_amd.profiling traffic FETCH_CSV WRITE_CSV --copy-mib 1024 \\
        --kernel gemm1=PATTERN --source FILE --workload NAME --command "..." > out.md
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
from collections import OrderedDict

COPY_KERNEL = "__amd_rocclr_copyBuffer"
TRAFFIC_TAG = "traffic-json:"


def short_name(kernel: str) -> str:
    """Kernel name without namespaces, argument list and return type."""
    k = kernel.replace("moe::(anonymous namespace)::", "").replace("void ", "")
    k = re.sub(r"\((moe::)?(\(anonymous namespace\)::)?[A-Za-z_][^()]*\)$", "", k)
    return k.strip()


def dispatch_medians(trace_csv: str) -> dict:
    """{kernel name: median duration in ns} over the dispatches of a
    ``--kernel-trace`` CSV (the mean of a short profiled run is pulled up by
    its first, cold launches)."""
    per = {}
    for r in csv.DictReader(open(trace_csv)):
        per.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = {}
    for name, d in per.items():
        d.sort()
        n = len(d)
        out[name] = d[n // 2] if n % 2 else 0.5 * (d[n // 2 - 1] + d[n // 2])
    return out


def summarize_trace(stats_csv: str, command: str, title: str, trace_csv: str = None) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    med = dispatch_medians(trace_csv) if trace_csv else None
    out = ["# %s" % title, "", "Command:", "", "```", command, "```", ""]
    if med is None:
        out += ["| kernel | calls | mean (us) | min (us) | max (us) | share of GPU time |",
                "|---|---:|---:|---:|---:|---:|"]
    else:
        out += ["| kernel | calls | mean (us) | median (us) | min (us) | max (us) | share of GPU time |",
                "|---|---:|---:|---:|---:|---:|---:|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        cells = [float(r["AverageNs"]) / 1e3]
        if med is not None:
            cells.append(med.get(r["Name"], float("nan")) / 1e3)
        cells += [float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3]
        out.append("| `%s` | %s | %s | %.1f %% |" % (
            short_name(r["Name"]), r["Calls"], " | ".join("%.1f" % c for c in cells),
            100.0 * float(r["TotalDurationNs"]) / total))
    return "\n".join(out) + "\n"


def _per_dispatch(counter_csv: str, counter: str):
    """{dispatch id: (kernel name, summed counter value)} in dispatch order."""
    per = OrderedDict()
    for r in csv.DictReader(open(counter_csv)):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        name, v = per.get(d, (r["Kernel_Name"], 0.0))
        per[d] = (name, v + float(r["Counter_Value"]))
    return per


def _copy_factor(per, copy_bytes: int) -> float:
    """Bytes per counter unit, from the largest copy kernel of the run."""
    vals = [v for name, v in per.values() if COPY_KERNEL in name]
    if not vals or max(vals) <= 0:
        raise ValueError("no calibration copy in the counter file")
    return copy_bytes / max(vals)


def file_sha256(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def summarize_traffic(fetch_csv: str, write_csv: str, copy_mib: int, kernels: dict, source: str,
                      workload: str, command: str, repo_root: str) -> str:
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    copy_bytes = copy_mib << 20
    ff, wf = _copy_factor(fetch, copy_bytes), _copy_factor(write, copy_bytes)
    result = {}
    lines = []
    for label, pattern in kernels.items():
        rx = re.compile(pattern)
        fv = [v for name, v in fetch.values() if rx.search(name)]
        wv = [v for name, v in write.values() if rx.search(name)]
        if not fv or not wv:
            raise ValueError("kernel %s (%s) not found" % (label, pattern))
        f_b = sum(fv) / len(fv) * ff
        w_b = sum(wv) / len(wv) * wf
        result[label] = {"read_bytes": round(f_b), "write_bytes": round(w_b), "bytes": round(f_b + w_b),
                         "launches": [len(fv), len(wv)]}
        lines.append("| %s | `%s` | %d / %d | %.4f | %.4f | %.4f |" % (
            label, pattern, len(fv), len(wv), f_b / 1e9, w_b / 1e9, (f_b + w_b) / 1e9))
    src_rel = os.path.relpath(source, repo_root)
    payload = {"workload": workload, "source": src_rel, "source_sha256": file_sha256(source),
               "fetch_bytes_per_unit": ff, "write_bytes_per_unit": wf, "kernels": result}
    out = ["# HBM traffic per launch: %s" % workload, "",
           "Commands (one counter pass each; the run also copies %d MiB device to device, whose counts "
           "give the scale of each counter):" % copy_mib, "", "```", command, "```", "",
           "Scale: FETCH_SIZE x %.1f bytes per unit, WRITE_SIZE x %.1f bytes per unit." % (ff, wf), "",
           "| kernel | name pattern | launches (fetch/write pass) | read GB | written GB | total GB |",
           "|---|---|---:|---:|---:|---:|"] + lines + [
           "", "Source measured: `%s` (sha256 %s). The benchmark reports these bytes only while that "
           "file is unchanged." % (src_rel, payload["source_sha256"][:16]), "",
           "%s %s" % (TRAFFIC_TAG, json.dumps(payload, sort_keys=True))]
    return "\n".join(out) + "\n"


def traffic_bytes(summary_md: str, label: str, repo_root: str):
    """HBM bytes per launch of kernel `label` from a traffic summary, or None
    when the summary is missing or its kernel source has changed since."""
    if not os.path.exists(summary_md):
        return None
    for line in open(summary_md):
        if line.startswith(TRAFFIC_TAG):
            payload = json.loads(line[len(TRAFFIC_TAG):])
            src = os.path.join(repo_root, payload["source"])
            if not os.path.exists(src) or file_sha256(src) != payload["source_sha256"]:
                return None
            k = payload["kernels"].get(label)
            return None if k is None else k["bytes"]
    return None


# Per-dispatch normalisation of the counters summarised by `counters`: what each
# counter's total is divided by to give a per-unit figure on the MI355X (8
# XCDs, 256 CUs, 1024 SIMDs). GRBM_GUI_ACTIVE sums the active cycles of the 8
# XCDs; SQ_VALU_MFMA_BUSY_CYCLES sums over the SIMDs; the SQ_WAIT_* and
# SQ_WAVE_CYCLES counters count wave-cycles in units of 4 cycles.
def derived_counters(tot: dict) -> "OrderedDict[str, float]":
    """Figures derived from one dispatch's counter totals (those available)."""
    out = OrderedDict()
    cycles = tot.get("GRBM_GUI_ACTIVE")
    if cycles:
        cyc = cycles / 8.0  # per XCD: the kernel's duration in GPU clocks
        out["clock cycles (GRBM_GUI_ACTIVE / 8)"] = cyc
        if "SQ_VALU_MFMA_BUSY_CYCLES" in tot:
            out["MFMA busy share (per SIMD)"] = tot["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024.0 / cyc
        if "SQ_INSTS_LDS_LOAD_BANDWIDTH" in tot:
            out["LDS bytes read per CU per clock"] = tot["SQ_INSTS_LDS_LOAD_BANDWIDTH"] * 64.0 / 256.0 / cyc
        if "SQ_LDS_CMD_FIFO_FULL" in tot:
            out["LDS command FIFO full share (per CU)"] = tot["SQ_LDS_CMD_FIFO_FULL"] / 256.0 / cyc
    if tot.get("SQ_WAVE_CYCLES"):
        for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS"):
            if c in tot:
                out["%s / SQ_WAVE_CYCLES" % c] = tot[c] / tot["SQ_WAVE_CYCLES"]
    return out


def summarize_counters(csvs: list, kernels: dict, workload: str, command: str) -> str:
    """Mean per-dispatch totals of every counter in the given --pmc CSVs for
    each kernel pattern, and the figures derived from them."""
    lines = ["# Counters per launch: %s" % workload, "", "Commands (one pass per CSV):", "", "```", command, "```", ""]
    for label, pattern in kernels.items():
        rx = re.compile(pattern)
        tot = OrderedDict()
        launches = {}
        for path in csvs:
            per = {}
            for r in csv.DictReader(open(path)):
                if not rx.search(r["Kernel_Name"]):
                    continue
                d = per.setdefault(r["Dispatch_Id"], {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            if not per:
                raise ValueError("kernel %s (%s) not found in %s" % (label, pattern, path))
            for c in sorted({c for d in per.values() for c in d}):
                vals = [d[c] for d in per.values() if c in d]
                if c in tot:  # the same counter in two passes (the clock): average them
                    tot[c] = 0.5 * (tot[c] + sum(vals) / len(vals))
                else:
                    tot[c] = sum(vals) / len(vals)
                launches[c] = len(vals)
        lines += ["## %s (`%s`)" % (label, pattern), "", "| counter | mean per launch | launches |", "|---|---:|---:|"]
        lines += ["| %s | %.4g | %d |" % (c, v, launches[c]) for c, v in tot.items()]
        lines += ["", "| derived | value |", "|---|---:|"]
        lines += ["| %s | %.4g |" % (k, v) for k, v in derived_counters(tot).items()]
        lines.append("")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("--command", required=True)
    t.add_argument("--title", default="Kernel trace")
    t.add_argument("--trace-csv", default=None, help="per-dispatch kernel trace CSV: adds a median column")
    f = sub.add_parser("traffic")
    f.add_argument("fetch_csv")
    f.add_argument("write_csv")
    f.add_argument("--copy-mib", type=int, required=True)
    f.add_argument("--kernel", action="append", required=True, metavar="LABEL=REGEX")
    f.add_argument("--source", required=True)
    f.add_argument("--workload", required=True)
    f.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--kernel", action="append", required=True, metavar="LABEL=REGEX")
    c.add_argument("--workload", required=True)
    c.add_argument("--command", required=True)
    a = ap.parse_args()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if a.what == "counters":
        print(summarize_counters(a.csv, OrderedDict(kv.split("=", 1) for kv in a.kernel), a.workload, a.command),
              end="")
        return
    if a.what == "trace":
        print(summarize_trace(a.stats_csv, a.command, a.title, a.trace_csv), end="")
    else:
        kernels = OrderedDict(kv.split("=", 1) for kv in a.kernel)
        print(summarize_traffic(a.fetch_csv, a.write_csv, a.copy_mib, kernels, a.source, a.workload, a.command,
                                root), end="")


if __name__ == "__main__":
    main()
