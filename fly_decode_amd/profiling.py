"""Summaries of rocprofv3 output for the benchmark's roofline block.

Two kinds of summary are written under ``profiles/`` (short text, nothing executable); the
benchmark calls them (``bench.py --summarize-trace`` and ``--summarize-traffic``):

* ``summarize_timed_trace``: the per-kernel and per-step figures of a ``rocprofv3 --kernel-trace``
  run of the benchmark, restricted to its timed steps, as markdown, with the command that produced
  it.
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


def _trace_rows(trace_dir: str):
    rows = []
    for p in _csvs(trace_dir, "kernel_trace.csv"):
        with open(p, newline="") as f:
            for r in csv.DictReader(f):
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), _short_name(r["Kernel_Name"])))
    if not rows:
        raise ValueError(f"no kernel_trace.csv under {trace_dir}")
    rows.sort()
    return rows


def summarize_timed_trace(trace_dir: str, line: dict, out_md: str, title: str, command: str,
                          peak_gbps: float = 8000.0):
    """Per-kernel and per-step figures of the benchmark's timed steps only.

    The library's dispatches (kernel names starting with ``k_``) are taken in start order; the last
    steps x launches_per_step of them are the timed steps (after the timed region the benchmark
    launches only copies).  Reports each kernel's mean duration over those dispatches, each step's
    summed kernel time and span (first start to last end), and the fraction of the HBM peak that the
    step's algorithmic bytes give over each, next to the fraction the JSON line reports."""
    cfg = line["config"]
    steps, per_step = int(line["steps"]), int(cfg["launches_per_step"])
    lib = [r for r in _trace_rows(trace_dir) if r[2].startswith("k_")]
    if len(lib) < steps * per_step:
        raise ValueError(f"{len(lib)} library dispatches, fewer than {steps} x {per_step}")
    timed = lib[-steps * per_step:]
    by_name = {}
    for s0, s1, name in timed:
        by_name.setdefault(name, []).append(s1 - s0)
    sums, spans = [], []
    for k in range(steps):
        chunk = timed[k * per_step:(k + 1) * per_step]
        sums.append(sum(s1 - s0 for s0, s1, _ in chunk))
        spans.append(chunk[-1][1] - chunk[0][0])
    step_bytes = float(cfg["compressed_bytes_per_step"])
    sum_ns, span_ns = statistics.fmean(sums), statistics.fmean(spans)
    lines = [f"# {title}", "",
             "Command (run from /tmp with TMPDIR=/tmp on one MI355X; committed files only):", "",
             "```", command, "```", "",
             f"Timed steps only: the last {steps} steps x {per_step} launches of the library's kernels "
             f"({len(lib)} library dispatches in the trace, warm-up included).", "",
             "| kernel | dispatches | mean ns | min ns | max ns |", "|---|---|---|---|---|"]
    for name, d in sorted(by_name.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{name}` | {len(d)} | {statistics.fmean(d):.0f} | {min(d)} | {max(d)} |")
    lines += ["", "| per step | mean | fraction of HBM peak from the step's algorithmic bytes |",
              "|---|---|---|",
              f"| summed kernel time | {sum_ns / 1e3:.2f} us | {step_bytes / sum_ns / peak_gbps:.4f} |",
              f"| span, first start to last end | {span_ns / 1e3:.2f} us | {step_bytes / span_ns / peak_gbps:.4f} |",
              f"| HIP events in the same run (the JSON line) | {float(line['ms_per_step']) * 1e3:.2f} us | "
              f"{line['roofline']['frac']:.4f} |", "",
              f"Algorithmic bytes per step: {int(step_bytes)} ({cfg['workload']}, {cfg['tensors']} tensors)."]
    # (a chained run is one launch per step: no per-phase dispatches to tabulate)
    pattern = cfg.get("phase_pattern") if cfg.get("launch", "phases") == "phases" else None
    if pattern:
        per = len(pattern)
        lines += ["", "Per launch of a layer (position in the repeating pattern):", "",
                  "| launch | tensors | algorithmic bytes | mean ns | fraction of HBM peak |", "|---|---|---|---|---|"]
        for j, (names, nbytes) in enumerate(pattern):
            d = [s1 - s0 for i, (s0, s1, _) in enumerate(timed) if (i % per_step) % per == j]
            m = statistics.fmean(d)
            lines.append(f"| {j} | {names} | {nbytes} | {m:.0f} | {nbytes / m / peak_gbps:.4f} |")
    os.makedirs(os.path.dirname(out_md), exist_ok=True)
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return {"sum_ns": sum_ns, "span_ns": span_ns}


def summarize_counters(run_dirs, kernel_prefix: str, out_md: str, title: str, command: str,
                       clock_ghz: float = 2.4, cus: int = 256):
    """Mean per dispatch of every counter in the ``--pmc`` runs under run_dirs, for the kernels whose
    short name starts with kernel_prefix, plus the ratios used to read them: the fraction of the
    dispatch's CU-cycles the LDS was busy (SQ_LDS_IDX_ACTIVE) and, of those, lost to bank conflicts
    (SQ_LDS_BANK_CONFLICT); the fraction of wave time spent waiting to issue (SQ_WAIT_INST_ANY, of
    which on the LDS queue: SQ_WAIT_INST_LDS) and waiting on dependencies (SQ_WAIT_ANY), both over
    SQ_WAVE_CYCLES; and instructions per wave."""
    vals, durs = {}, []
    for d in run_dirs:
        for p in _csvs(d, "counter_collection.csv"):
            with open(p, newline="") as f:
                for r in csv.DictReader(f):
                    if not _short_name(r["Kernel_Name"]).startswith(kernel_prefix):
                        continue
                    vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                    if r["Counter_Name"] == "SQ_WAVES":
                        durs.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    if not vals:
        raise ValueError(f"no counter samples for {kernel_prefix!r}")
    m = {k: statistics.fmean(v) for k, v in vals.items()}
    lines = [f"# {title}", "", "Commands (run from /tmp with TMPDIR=/tmp on one MI355X; committed files only):", "",
             "```", command, "```", "",
             f"Mean per dispatch over the dispatches of kernels named `{kernel_prefix}*` "
             f"({len(vals.get('SQ_WAVES', []))} in the SQ pass).", "",
             "| counter | mean per dispatch |", "|---|---|"]
    for k in sorted(m):
        lines.append(f"| `{k}` | {m[k]:.1f} |")
    derived = []
    if durs:
        cyc = statistics.fmean(durs) * clock_ghz  # ns * GHz = cycles
        derived.append(("mean dispatch duration", f"{statistics.fmean(durs) / 1e3:.2f} us"))
        if "SQ_LDS_IDX_ACTIVE" in m:
            derived.append(("LDS busy, fraction of the dispatch's CU-cycles", f"{m['SQ_LDS_IDX_ACTIVE'] / cus / cyc:.3f}"))
    if "SQ_LDS_BANK_CONFLICT" in m and "SQ_LDS_IDX_ACTIVE" in m:
        derived.append(("bank-conflict cycles over LDS busy cycles", f"{m['SQ_LDS_BANK_CONFLICT'] / m['SQ_LDS_IDX_ACTIVE']:.3f}"))
    if "SQ_WAVE_CYCLES" in m:
        for c, what in (("SQ_WAIT_INST_ANY", "waiting to issue"), ("SQ_WAIT_INST_LDS", "waiting to issue to the LDS"),
                        ("SQ_WAIT_ANY", "waiting on dependencies")):
            if c in m:
                derived.append((f"wave time {what}", f"{m[c] / m['SQ_WAVE_CYCLES']:.3f}"))
    if "SQ_WAVES" in m:
        for c in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_MFMA"):
            if c in m:
                derived.append((f"{c} per wave", f"{m[c] / m['SQ_WAVES']:.0f}"))
    if derived:
        lines += ["", "| derived | value |", "|---|---|"] + [f"| {a} | {b} |" for a, b in derived]
    os.makedirs(os.path.dirname(out_md), exist_ok=True)
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return m
