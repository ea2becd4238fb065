"""Summaries of rocprofv3 output for the committed profile records.

Reads rocprofv3 CSV output (``--kernel-trace --stats -f csv`` and
``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs of bench.py with
``--copy-calibration``) and writes:

* ``<kernel>_<workload>.md``: average duration per kernel from the stats,
  with the command that produced them, and the dominant kernel's average
  over its last ``--steps`` launches (the bench's timed launches follow its
  warm-up ones, which run while the GPU clock is still rising);
* ``<kernel>_<workload>_counters.json``: HBM bytes per launch of the
  dominant kernel, each counter scaled by what it reads for the plain
  1 GiB device copy (``__amd_rocclr_copyBuffer``) of the same run, and the
  hash of the kernel source it was measured on (bench.py reports the
  traffic only while that hash matches).

Usage: python -m subquadratic_attention_amd.prof <name> <workload> <kernel-substring>
       <source> <trace_dir> <fetch_dir> <write_dir> <out_dir> <command...>
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys

COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30


def _rows(d: str, pattern: str):
    files = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if not files:
        raise FileNotFoundError(f"no {pattern} under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def counter_values(d: str):
    acc = {}
    for r in _rows(d, "*counter_collection.csv"):
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return acc


def pick(values, sub, how="mean"):
    hits = [k for k in values if sub in k]
    if not hits:
        raise KeyError(sub)
    v = values[hits[0]]
    return max(v) if how == "max" else sum(v) / len(v)


def timed_average_us(trace_dir: str, sub: str, command: str):
    """(launches, average in us) of the last --steps launches of the kernel
    matching sub in the kernel trace, or None without --steps."""
    words = command.split()
    if "--steps" not in words:
        return None
    k = int(words[words.index("--steps") + 1])
    rows = [r for r in _rows(trace_dir, "*kernel_trace.csv") if sub in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    last = rows[-k:]
    if not last:
        return None
    return len(last), sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in last) / len(last) / 1e3


def source_hash(root: str, rel: str) -> str:
    with open(os.path.join(root, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def main(argv):
    name, workload, ksub, source, trace_dir, fetch_dir, write_dir, out_dir = argv[:8]
    command = " ".join(argv[8:])
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    stats = _rows(trace_dir, "*kernel_stats.csv")
    lines = [f"# {name}: {workload}", "", "Produced by:", "", "```", command, "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    timed = timed_average_us(trace_dir, ksub, command.split(";")[0])
    if timed is not None:
        lines += ["", f"Dominant kernel, its last {timed[0]} launches in this trace (--steps of the traced "
                  f"command): average {timed[1]:.2f} us."]
    fetch = counter_values(fetch_dir)
    write = counter_values(write_dir)
    # the calibration copy is the largest device copy of the run
    f_scale = COPY_BYTES / (pick(fetch, COPY_KERNEL, "max") * 1024)
    w_scale = COPY_BYTES / (pick(write, COPY_KERNEL, "max") * 1024)
    kf = pick(fetch, ksub) * 1024 * f_scale
    kw = pick(write, ksub) * 1024 * w_scale
    lines += ["", "HBM traffic of the dominant kernel (rocprofv3 `--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`, "
              "each in its own run, scaled by the same counter on a plain 1 GiB device copy):", "",
              f"- FETCH_SIZE scale factor (1 GiB / copy's FETCH_SIZE): {f_scale:.3f}",
              f"- WRITE_SIZE scale factor (1 GiB / copy's WRITE_SIZE): {w_scale:.3f}",
              f"- read bytes per launch: {kf:.4g}", f"- written bytes per launch: {kw:.4g}",
              f"- source hash of `{source}`: {source_hash(root, source)}"]
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"{name}_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    rec = {"kernel": ksub, "workload": workload, "source": source, "source_hash": source_hash(root, source),
           "fetch_scale": f_scale, "write_scale": w_scale, "read_bytes_per_launch": kf,
           "write_bytes_per_launch": kw, "hbm_bytes_per_launch": kf + kw, "command": command}
    with open(os.path.join(out_dir, f"{name}_{workload}_counters.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


if __name__ == "__main__":
    main(sys.argv[1:])
