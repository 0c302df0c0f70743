"""Summaries of rocprofv3 output for the benchmark's roofline block.

Two kinds of summary are written under ``profiles/`` (short text, nothing executable):

* ``summarize_trace``: the per-kernel table of a ``rocprofv3 --kernel-trace --stats`` run
  (``*_kernel_stats.csv``), as markdown, with the command that produced it.
* ``summarize_traffic``: HBM bytes per dispatch of one kernel from two ``--pmc`` runs (``FETCH_SIZE``,
  then ``WRITE_SIZE``), each scaled by what the same counter reads for a plain device-to-device copy
  of known size (``bench.py --copy-calibration``).  The JSON records the SHA-256 of the kernel
  source it was measured on; ``traffic_for`` returns the figure only while that source is unchanged.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fly_decode_amd", "csrc")
KERNEL_SOURCE = os.path.join(CSRC, "cbk_kernels.hip")
ENCODER_SOURCE = os.path.join(CSRC, "cbk_encode.hip")
EC_SOURCE = os.path.join(CSRC, "cbk_ec.hip")
PROFILES = os.path.join(ROOT, "profiles")


def source_for(kernel: str) -> str:
    """The source file that defines a kernel: the GPU encoder's are named k_enc_*, the entropy-coded
    format's k_ec_*, the rest live in cbk_kernels.hip."""
    if kernel.startswith("k_enc"):
        return ENCODER_SOURCE
    if kernel.startswith("k_ec"):
        return EC_SOURCE
    return KERNEL_SOURCE


def kernel_source_sha256(kernel: str = "") -> str:
    with open(source_for(kernel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _short_name(name: str) -> str:
    """`void cbk::(anonymous namespace)::k_gemv_rows<13>(...)` -> `k_gemv_rows<13>`."""
    base = name.replace("(anonymous namespace)", "anon").split("(")[0]
    if "::" in base:
        base = base.split("::")[-1]
    return base.replace("void ", "").strip()


def _csvs(path: str, suffix: str):
    if os.path.isfile(path):
        return [path]
    return sorted(glob.glob(os.path.join(path, "**", "*" + suffix), recursive=True))


def counter_per_dispatch(run_dir: str, counter: str, kernel_prefix: str):
    """Mean and count of `counter` over the dispatches whose short kernel name starts with
    `kernel_prefix`, from the counter_collection CSV(s) under `run_dir`."""
    vals = []
    for p in _csvs(run_dir, "counter_collection.csv"):
        with open(p, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                if _short_name(r["Kernel_Name"]).startswith(kernel_prefix):
                    vals.append(float(r["Counter_Value"]))
    if not vals:
        raise ValueError(f"no {counter} samples for kernels starting with {kernel_prefix!r} in {run_dir}")
    return statistics.fmean(vals), len(vals)


def summarize_traffic(out_json: str, kernel_prefix: str, fetch_dir: str, write_dir: str,
                      copy_fetch_dir: str, copy_write_dir: str, copy_bytes: int,
                      algorithmic_bytes: float, command: str, copy_kernel_prefix: str = "__amd_rocclr_copyBuffer",
                      dispatches_per_unit: int = 1):
    """Traffic per unit of work: the mean counter value over the matching dispatches times
    `dispatches_per_unit` (a unit that is several different kernels, one dispatch each, sums them)."""
    f_k, n_f = counter_per_dispatch(fetch_dir, "FETCH_SIZE", kernel_prefix)
    w_k, n_w = counter_per_dispatch(write_dir, "WRITE_SIZE", kernel_prefix)
    f_c, _ = counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE", copy_kernel_prefix)
    w_c, _ = counter_per_dispatch(copy_write_dir, "WRITE_SIZE", copy_kernel_prefix)
    # scale: bytes per counter unit, from the copy of known size (reads copy_bytes, writes copy_bytes)
    fetch_scale, write_scale = copy_bytes / f_c, copy_bytes / w_c
    read_b, write_b = f_k * fetch_scale * dispatches_per_unit, w_k * write_scale * dispatches_per_unit
    rec = {
        "kernel": kernel_prefix,
        "dispatches_per_unit": dispatches_per_unit,
        "source_sha256": kernel_source_sha256(kernel_prefix),
        "fetch_size_per_dispatch": f_k, "fetch_dispatches": n_f,
        "write_size_per_dispatch": w_k, "write_dispatches": n_w,
        "copy_bytes": copy_bytes, "copy_fetch_size": f_c, "copy_write_size": w_c,
        "fetch_bytes_per_unit": fetch_scale, "write_bytes_per_unit": write_scale,
        "read_bytes_per_launch": read_b, "write_bytes_per_launch": write_b,
        "traffic_bytes_per_launch": read_b + write_b,
        "algorithmic_bytes_per_launch": algorithmic_bytes,
        "traffic_over_algorithmic": (read_b + write_b) / algorithmic_bytes if algorithmic_bytes else None,
        "command": command,
    }
    os.makedirs(os.path.dirname(out_json), exist_ok=True)
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def traffic_path(kernel_key: str, workload: str) -> str:
    return os.path.join(PROFILES, f"traffic_{kernel_key}_{workload}.json")


def traffic_for(kernel_key: str, workload: str):
    """The traffic record for this kernel and workload, or None when none exists or the kernel
    source has changed since the counters were taken."""
    p = traffic_path(kernel_key, workload)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_source_sha256(kernel_key):
        return None
    return rec


def summarize_trace(stats_csv: str, out_md: str, title: str, command: str, notes: str = ""):
    rows = []
    for p in _csvs(stats_csv, "kernel_stats.csv"):
        with open(p, newline="") as f:
            for r in csv.DictReader(f):
                rows.append(r)
    if not rows:
        raise ValueError(f"no kernel_stats.csv under {stats_csv}")
    lines = [f"# {title}", "", "Command (run from /tmp with TMPDIR=/tmp on one MI355X; committed files only):", "",
             "```", command, "```", "", "Kernel statistics (`kernel_stats.csv`):", "",
             "| kernel | calls | average ns | min ns | max ns | share |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r.get("Percentage", 0) or 0)):
        lines.append(f"| `{_short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                     f"{float(r['MinNs']):.0f} | {float(r['MaxNs']):.0f} | {float(r['Percentage']):.2f} % |")
    if notes:
        lines += ["", notes]
    os.makedirs(os.path.dirname(out_md), exist_ok=True)
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return rows
