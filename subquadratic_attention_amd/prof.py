"""Summaries of rocprofv3 output for the committed profile records.

Reads rocprofv3 CSV output (``--kernel-trace --stats -f csv`` and
``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs of ``bench.py --only <leg>``
with ``--copy-calibration``) and writes:

* ``<name>_<workload>.md``: the per-kernel statistics of the trace, with the
  command that produced them, and for each kernel of the leg's step its
  average over the leg's timed launches.  In a ``--only`` run of bench.py a
  leg times its step last, so those are the last ``timed`` launches of each
  such kernel in the trace (each kernel of the benchmark workloads runs once
  per step); ``timed`` is the leg's own count of timed steps, printed in its
  JSON record (``timed_steps``);
* ``<name>_<workload>_counters.json``: HBM bytes per launch of each kernel of
  the step and their sum per step, each counter scaled by what it reads for
  the plain 1 GiB device copy (``__amd_rocclr_copyBuffer``) of the same run,
  and the hash of the kernel source they were measured on (bench.py reports
  the traffic only while that hash matches).

Usage: python -m subquadratic_attention_amd.prof <name> <workload>
       <kernel-substring[,kernel-substring...]> <source[,source...]> <trace_dir>
       <fetch_dir> <write_dir> <out_dir> <timed> <command...>

With ``sq`` first, it summarises two SQ counter runs (``--pmc`` of the
instruction counters, then of the busy / wait cycle counters) into
``<name>_<workload>_sq.md``: per kernel, instructions per wavefront by kind,
and MFMA, VALU and LDS activity as fractions of the kernel's cycles:

       python -m subquadratic_attention_amd.prof sq <name> <workload>
       <kernel-substring[,...]> <insts_dir> <cycles_dir> <out_dir> <command...>
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


def _match(names, sub):
    hits = sorted(k for k in names if sub in k)
    if not hits:
        raise KeyError(sub)
    if len(hits) > 1:
        raise KeyError(f"{sub} matches {len(hits)} kernels: {hits}")
    return hits[0]


def pick(values, sub, how="mean"):
    v = values[_match(values, sub)]
    return max(v) if how == "max" else sum(v) / len(v)


def timed_average_us(trace_dir: str, sub: str, timed: int):
    """(launches, average in us) of the last `timed` launches of the kernel
    matching sub in the kernel trace."""
    rows = [r for r in _rows(trace_dir, "*kernel_trace.csv") if sub in r["Kernel_Name"]]
    names = {r["Kernel_Name"] for r in rows}
    if len(names) != 1:
        raise KeyError(f"{sub} matches {sorted(names)}")
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    last = rows[-timed:]
    return len(last), sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in last) / len(last) / 1e3


def source_hash(root: str, rels: str) -> str:
    """Hash of the kernel sources (comma-separated paths, in order)."""
    h = hashlib.sha256()
    for rel in rels.split(","):
        with open(os.path.join(root, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def main(argv):
    name, workload, ksubs, source, trace_dir, fetch_dir, write_dir, out_dir, timed = argv[:9]
    subs = ksubs.split(",")
    timed = int(timed)
    command = " ".join(argv[9:])
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    stats = _rows(trace_dir, "*kernel_stats.csv")
    lines = [f"# {name}: {workload}", "", "Produced by:", "", "```", command, "```", "",
             "All calls of each kernel in the traced process (warm-up included):", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    lines += ["", f"The leg's timed launches (its last {timed} launches of each kernel of its step; the leg's record "
              f"says timed_steps = {timed}):", "", "| kernel | launches | average (us) |", "|---|---|---|"]
    total_us = 0.0
    for sub in subs:
        n, avg = timed_average_us(trace_dir, sub, timed)
        total_us += avg
        lines.append(f"| `{sub}` | {n} | {avg:.2f} |")
    if len(subs) > 1:
        lines.append(f"| sum per step | | {total_us:.2f} |")
    fetch = counter_values(fetch_dir)
    write = counter_values(write_dir)
    # the calibration copy is the largest device copy of the run
    f_scale = COPY_BYTES / (pick(fetch, COPY_KERNEL, "max") * 1024)
    w_scale = COPY_BYTES / (pick(write, COPY_KERNEL, "max") * 1024)
    per = {}
    for sub in subs:
        per[sub] = {"read_bytes_per_launch": pick(fetch, sub) * 1024 * f_scale,
                    "write_bytes_per_launch": pick(write, sub) * 1024 * w_scale}
    tr = sum(v["read_bytes_per_launch"] for v in per.values())
    tw = sum(v["write_bytes_per_launch"] for v in per.values())
    lines += ["", "HBM traffic per launch (rocprofv3 `--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`, each in its own run, "
              "scaled by the same counter on a plain 1 GiB device copy):", "",
              f"- FETCH_SIZE scale factor (1 GiB / copy's FETCH_SIZE): {f_scale:.3f}",
              f"- WRITE_SIZE scale factor (1 GiB / copy's WRITE_SIZE): {w_scale:.3f}", "",
              "| kernel | read bytes | written bytes |", "|---|---|---|"]
    for sub, v in per.items():
        lines.append(f"| `{sub}` | {v['read_bytes_per_launch']:.4g} | {v['write_bytes_per_launch']:.4g} |")
    if len(subs) > 1:
        lines.append(f"| sum per step | {tr:.4g} | {tw:.4g} |")
    lines += ["", f"Source hash of `{source}`: {source_hash(root, source)}"]
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"{name}_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    rec = {"kernels": per, "workload": workload, "source": source, "source_hash": source_hash(root, source),
           "fetch_scale": f_scale, "write_scale": w_scale, "timed_steps": timed,
           "read_bytes_per_launch": tr, "write_bytes_per_launch": tw, "hbm_bytes_per_launch": tr + tw,
           "command": command}
    with open(os.path.join(out_dir, f"{name}_{workload}_counters.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


# The kernel's duration in GPU cycles is GRBM_GUI_ACTIVE / 8 (one GRBM per
# XCD, summed): checked against the traced duration at 2.4 GHz.
# SQ_VALU_MFMA_BUSY_CYCLES counts SIMD cycles of matrix-core work (16 per
# 16x16x32 bf16 MFMA: it equals 16 x SQ_INSTS_MFMA for the bf16 kernels);
# SQ_ACTIVE_INST_VALU / _LDS count, summed over the waves, the quad-cycles
# (4 cycles) in which a wave issues that kind of instruction;
# SQ_LDS_BANK_CONFLICT counts CU cycles stalled on LDS bank conflicts;
# SQ_WAIT_INST_ANY and SQ_WAVE_CYCLES count quad-cycles summed over waves.
INSTS = ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD",
         "SQ_INSTS_VMEM_WR", "SQ_INSTS_VALU_TRANS_F32"]
CYCLES = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
          "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_ANY", "GRBM_GUI_ACTIVE"]
CUS, SIMDS, XCDS = 256, 4, 8


def counters_by_kernel(d: str):
    """{kernel name: {counter: mean over the kernel's dispatches}}."""
    acc = {}
    for r in _rows(d, "*counter_collection.csv"):
        acc.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


def sq_main(argv):
    name, workload, ksubs, insts_dir, cycles_dir, out_dir = argv[:6]
    command = " ".join(argv[6:])
    a = counters_by_kernel(insts_dir)
    b = counters_by_kernel(cycles_dir)
    lines = [f"# {name}: {workload}, SQ counters", "", "Produced by:", "", "```", command, "```", "",
             "Each value is the mean over the kernel's dispatches in that run.  Instructions are per "
             "wavefront (SQ_INSTS_* / SQ_WAVES).  With T = GRBM_GUI_ACTIVE / 8 the kernel's cycles (one GRBM per "
             "XCD): MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (T x 1024 SIMDs), the share of SIMD cycles the matrix "
             "cores work; VALU issue = 4 SQ_ACTIVE_INST_VALU / (T x 1024), the share of SIMD cycles issuing VALU "
             "instructions (summed over the SIMD's waves); LDS issue likewise from SQ_ACTIVE_INST_LDS; LDS "
             "conflict = SQ_LDS_BANK_CONFLICT / (T x 256 CUs), the share of CU cycles stalled on bank conflicts; "
             "waiting = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES, the share of resident-wave time spent waiting for "
             "outstanding memory or LDS results.", "",
             "| kernel | waves | VALU | (transc.) | MFMA | LDS | SALU | VMEM rd | VMEM wr | T (us at 2.4 GHz) | "
             "MFMA busy | VALU issue | LDS issue | LDS conflict | waiting |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    rec = {}
    for sub in ksubs.split(","):
        ka = _match(a, sub)
        kb = _match(b, sub)
        x, y = a[ka], b[kb]
        waves = x["SQ_WAVES"]
        per = {c: x[c] / waves for c in INSTS[1:]}
        T = y["GRBM_GUI_ACTIVE"] / XCDS
        mfma = y["SQ_VALU_MFMA_BUSY_CYCLES"] / (T * CUS * SIMDS)
        valu = 4 * y["SQ_ACTIVE_INST_VALU"] / (T * CUS * SIMDS)
        lds = 4 * y["SQ_ACTIVE_INST_LDS"] / (T * CUS * SIMDS)
        conf = y["SQ_LDS_BANK_CONFLICT"] / (T * CUS)
        wait = y["SQ_WAIT_INST_ANY"] / max(y["SQ_WAVE_CYCLES"], 1.0)
        lines.append(f"| `{sub}` | {waves:.0f} | {per['SQ_INSTS_VALU']:.0f} | {per['SQ_INSTS_VALU_TRANS_F32']:.0f} | "
                     f"{per['SQ_INSTS_MFMA']:.0f} | {per['SQ_INSTS_LDS']:.0f} | {per['SQ_INSTS_SALU']:.0f} | "
                     f"{per['SQ_INSTS_VMEM_RD']:.0f} | {per['SQ_INSTS_VMEM_WR']:.0f} | {T / 2400:.1f} | "
                     f"{100 * mfma:.1f} % | {100 * valu:.1f} % | {100 * lds:.1f} % | {100 * conf:.1f} % | "
                     f"{100 * wait:.1f} % |")
        rec[sub] = {"per_wave": per, "waves": waves, "cycles": T, "mfma_busy": mfma, "valu_issue": valu,
                    "lds_issue": lds, "lds_conflict": conf, "waiting": wait, "raw_insts": x, "raw_cycles": y}
    lines += ["", "Raw counter means per dispatch:", ""]
    for sub, r in rec.items():
        lines.append(f"- `{sub}`: " + ", ".join(f"{c} = {v:.4g}" for c, v in {**r['raw_insts'], **r['raw_cycles']}.items()))
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"{name}_{workload}_sq.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({k: {kk: vv for kk, vv in v.items() if not kk.startswith("raw")} for k, v in rec.items()}))


if __name__ == "__main__":
    if sys.argv[1:2] == ["sq"]:
        sq_main(sys.argv[2:])
    else:
        main(sys.argv[1:])
