#!/usr/bin/env python3
"""Benchmark: fused codebook-GEMV decompressed-weight GB/s at batch 1; % of HBM peak.

One step = one pass of the fused decode + GEMV (or skinny GEMM) over every tensor of the workload,
with the compressed tensors already resident in HBM.  Workloads (seeded synthetic BF16 weights,
each tensor with its own codebook):

  l70b_b1    (default) the 70B-shaped decode step at batch 1: 80 distinct layers of q/o 8192x8192,
             k/v 1024x8192, gate/up 28672x8192 and down 8192x28672, N(0, 0.015) (560 tensors,
             about 111 GB compressed, resident together).  Per layer four dependent phases:
             [q, k, v] and [gate, up] each one cbk_gemv_group launch (they share their input),
             o and down one cbk_gemv launch each.  --layers L times the first L layers instead.
  l70b_b16   the same step at batch 16 (cbk_gemm_group / cbk_gemm_small on the matrix cores).
  llama7b    the 7B-shaped decode step: 32 layers of q/k/v/o 4096x4096, gate/up 11008x4096 and
             down 4096x11008, N(0, 0.02) (224 tensors, 10.5 GB), phases as in l70b_b1.
  mlp_b1     the Llama-7B MLP at batch 1: gate/up 11008x4096 and down 4096x11008, 0.02 * t(4),
             --layers distinct copies (default 8, 1.76 GB, well past the 256 MB Infinity Cache);
             per layer [gate, up] one grouped launch, then down.
  mlp_b8     the same tensors at batch 8 (VALU skinny GEMM).
  attn4096   24 distinct 4096x4096 attention projections, N(0, 0.02), one cbk_gemv launch each.
  decode4096 standalone decode to BF16 in HBM of the attn4096 tensors, four per call
             (cbk_decode_group, a layer's [q, k, v, o]).
  ecdecode4096 / ecgemv4096  the attn4096 tensors in the exponent entropy-coded format, decoded to
             HBM (cbk_ec_decode_group, four tensors per launch, a layer's [q, k, v, o]) or decoded
             inside the batch-1 GEMV (cbk_ec_gemv_group, three per launch, a layer's [q, k, v]);
             --ec-index adds the span index.
  encode4096 cbk_encode_gpu_group of the attn4096 tensors from raw BF16 in HBM, four per call
             (three launches per call).
  --tensors-per-call G sets the tensors per call of these five (1: one call per tensor, as
  attn4096 always does by default).

The step workloads (l70b_*, llama7b) draw their weights on the GPU with the counter-based
generator of ``synth.counter`` and compress them there with cbk_encode_gpu, one tensor at a time,
so that 68 billion weights are ready in seconds; the other workloads draw on the host and upload.

Timing: untimed warm-up for --warmup steps and at least --warmup-seconds of wall time (the GPU
raises its clocks over the first tens of milliseconds of load), then --steps timed steps, each
bracketed by its own pair of HIP events on the launch stream (one HIP graph replay per step);
`ms_per_step` is their mean, `step_ms` their median, p10 and p90.  The timed region is bracketed by
torch.cuda.synchronize().  `value` = sum over the step of 2*rows*cols (the BF16 bytes the decode
feeds the multiply) / step time.  The roofline block uses the algorithmic bytes of the step's
launches (packed indices ceil(n*b/8) + codebook 2U + X 2*batch*K per launch + Y 4*batch*M) over
their time.  A device-to-device copy measured in the same run gives the copy bandwidth.

The CPU baseline (the oracle, decode + GEMV in float64) runs on sampled rows of every tensor of
the step, on the host threads the run may use and on one thread; its results for those rows are
compared with the GPU's output of the last timed step (the run fails on a mismatch).

Other modes: --summarize-trace and --summarize-traffic turn rocprofv3 output into the summaries
kept under profiles/; --copy-calibration runs the copy the traffic figures are scaled by.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
TOL = 1e-3  # |y - y_ref| <= TOL * sum_k |W x| per element
# tensors per call of the 4096x4096 workloads (--tensors-per-call overrides)
PER_CALL_DEFAULT = {"attn4096": 1, "decode4096": 4, "encode4096": 4, "ecdecode4096": 4, "ecgemv4096": 3}
STEP_WORKLOADS = ("l70b_b1", "l70b_b16", "llama7b")
ALL_WORKLOADS = ["l70b_b1", "l70b_b16", "llama7b", "mlp_b1", "mlp_b8", "attn4096", "decode4096",
                 "encode4096", "ecdecode4096", "ecgemv4096"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def host_threads() -> int:
    """Host threads this run may use: the CPUs it is allowed to run on, at most 16 (one GPU's
    share of a shared host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


# ------------------------------------------------------------------------------------ workloads

def workload_specs(name: str, count: int, layers: int):
    """(specs, phases, batch, layer_count): specs are (cfg, layer, tensor) triples; phases are lists
    of spec indices launched together (one launch per phase, phases run in order)."""
    import synth
    if name in ("attn4096", "decode4096", "encode4096", "ecdecode4096", "ecgemv4096"):
        t = synth.WORKLOADS[2][0][0]
        specs = [(2, layer, t) for layer in range(count)]
        return specs, [[i] for i in range(len(specs))], (1 if name in ("attn4096", "ecgemv4096") else 0), len(specs)
    if name in STEP_WORKLOADS:
        cfg = 4 if name == "llama7b" else 5
        tensors, n_layers = synth.WORKLOADS[cfg]
        n_layers = min(n_layers, layers) if layers else n_layers
        specs, phases = [], []
        names = [t.name for t in tensors]
        for layer in range(n_layers):
            base = len(specs)
            specs += [(cfg, layer, t) for t in tensors]
            for group in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
                phases.append([base + names.index(g) for g in group])
        return specs, phases, (16 if name == "l70b_b16" else 1), n_layers
    if name in ("mlp_b1", "mlp_b8"):
        tensors, _ = synth.WORKLOADS[3]
        layers = layers or 8
        specs = [(3, layer, t) for layer in range(layers) for t in tensors]
        # per layer: [gate, up] share their input (one grouped launch), then down
        phases = [p for l in range(layers) for p in ([3 * l, 3 * l + 1], [3 * l + 2])]
        return specs, phases, (8 if name == "mlp_b8" else 1), layers
    raise SystemExit(f"unknown workload {name}")


def prepare(specs, threads, cap=None, on_device=None):
    """Generate and compress every tensor, leaving the compressed forms on the GPU.  Tensors of
    the counter-based generator are drawn on the GPU and compressed by cbk_encode_gpu (no host
    copy); the others are drawn and compressed on the host (threads) and uploaded."""
    import torch
    import synth
    import fly_decode_amd as cbk

    if on_device is None:
        on_device = cap is None and all(t.dist == "normal_ctr" for _, _, t in specs)
    out = []
    if on_device:
        nmax = max(t.rows * t.cols for _, _, t in specs)
        raw = torch.empty(nmax, dtype=torch.int16, device="cuda")
        ws = torch.empty(cbk.encode_gpu_workspace_bytes(), dtype=torch.uint8, device="cuda")
        cb = torch.empty(65536, dtype=torch.int16, device="cuda")
        words = torch.empty(cbk.words_for(nmax, 16), dtype=torch.int32, device="cuda")
        meta = torch.zeros(2, dtype=torch.int32, device="cuda")
        for i, (cfg, layer, t) in enumerate(specs):
            n = t.rows * t.cols
            w = synth.workload_tensor_device(cfg, layer, t, "cuda", out=raw[:n])
            cbk.encode_gpu_launch(w, ws, cb, words, meta)
            U, b = (int(v) for v in meta.cpu().tolist())
            out.append(cbk.Compressed(t.rows, t.cols, U, b, cb[:U].clone(),
                                      words[:cbk.words_for(n, b)].clone()))
            if (i + 1) % 56 == 0 or i + 1 == len(specs):
                log(f"generated + encoded on the GPU {i + 1}/{len(specs)} tensors")
        del raw, ws, cb, words, meta
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        return out

    def make(spec):
        cfg, layer, t = spec
        return cbk.encode(synth.workload_tensor(cfg, layer, t), cap=cap)

    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        for i, c in enumerate(ex.map(make, specs)):
            out.append(c.to("cuda"))
            if (i + 1) % 16 == 0 or i + 1 == len(specs):
                log(f"encoded on the host + uploaded {i + 1}/{len(specs)} tensors")
    return out


class Workload:
    """A workload's tensors, inputs and outputs on the GPU, and its step (one pass of every phase's
    launch, in order), built exactly as the benchmark times it."""

    def __init__(self, name, count=24, layers=0, threads=None, cap=None, tensors=None, ec_index=False, per_call=0):
        import torch
        import synth
        import fly_decode_amd as cbk

        self.name = name
        self.specs, self.phases, self.batch, self.n_layers = workload_specs(name, count, layers)
        self.encode = name == "encode4096"
        self.ecfmt = name in ("ecdecode4096", "ecgemv4096")
        self.ecgemv = name == "ecgemv4096"
        if name in PER_CALL_DEFAULT:
            # tensors per call: a layer's [q, k, v, o] decoded or encoded together, the [q, k, v]
            # that share x in the entropy-coded fused GEMV; attn4096 is the single-tensor GEMV
            g = per_call or PER_CALL_DEFAULT[name]
            self.phases = [list(range(i, min(i + g, len(self.specs)))) for i in range(0, len(self.specs), g)]
        threads = threads or host_threads()
        t0 = time.perf_counter()
        if tensors is not None:
            self.tensors = tensors
        elif self.ecfmt:
            def make_ec(spec):
                cfg, layer, t = spec
                return cbk.ec_encode(synth.workload_tensor(cfg, layer, t))
            with cf.ThreadPoolExecutor(max_workers=threads) as ex:
                self.tensors = [e.to("cuda") for e in ex.map(make_ec, self.specs)]
        elif self.encode:
            def make_raw(spec):
                cfg, layer, t = spec
                w = synth.workload_tensor(cfg, layer, t)
                return w, cbk.encode(w)
            with cf.ThreadPoolExecutor(max_workers=threads) as ex:
                pairs = list(ex.map(make_raw, self.specs))
            self.raws = [torch.from_numpy(w.reshape(-1).view(np.int16)).to("cuda") for w, _ in pairs]
            # the host encodings: sizes for the byte count, and the check after timing
            self.tensors = [c for _, c in pairs]
            # one workspace per tensor of a run of up to 8
            self.ws = torch.empty(8 * cbk.encode_gpu_workspace_bytes(), dtype=torch.uint8, device="cuda")
            self.enc_cb = [torch.empty(65536, dtype=torch.int16, device="cuda") for _ in self.raws]
            self.enc_words = [torch.empty(cbk.words_for(r.numel(), 16), dtype=torch.int32, device="cuda")
                              for r in self.raws]
            self.enc_meta = [torch.zeros(2, dtype=torch.int32, device="cuda") for _ in self.raws]
        else:
            self.tensors = prepare(self.specs, threads, cap=cap)
        # the span index of the entropy-coded tensors (load-time work, outside the timed step)
        self.ec_index = [cbk.ec_build_index(t) for t in self.tensors] if (self.ecfmt and ec_index) else None
        self.setup_s = time.perf_counter() - t0

        self.xs = {}
        if self.batch > 0:
            for d in self.tensors:
                if d.cols not in self.xs:
                    x = synth.workload_x(self.specs[0][0], d.cols, self.batch)
                    self.xs[d.cols] = torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16)
        if self.encode:
            self.ys = []
        elif self.batch == 0:
            self.ys = [torch.empty((d.rows, d.cols), dtype=torch.bfloat16, device="cuda") for d in self.tensors]
        elif self.batch == 1:
            self.xs = {k: v[0] for k, v in self.xs.items()}
            self.ys = [torch.empty(d.rows, dtype=torch.float32, device="cuda") for d in self.tensors]
        else:
            self.ys = [torch.empty((self.batch, d.rows), dtype=torch.float32, device="cuda") for d in self.tensors]

    def step(self):
        import fly_decode_amd as cbk
        T, xs, ys = self.tensors, self.xs, self.ys
        for ph in self.phases:
            if self.encode and len(ph) == 1:
                i = ph[0]
                cbk.encode_gpu_launch(self.raws[i], self.ws, self.enc_cb[i], self.enc_words[i], self.enc_meta[i])
            elif self.encode:
                cbk.encode_gpu_group_launch([self.raws[i] for i in ph], self.ws, [self.enc_cb[i] for i in ph],
                                            [self.enc_words[i] for i in ph], [self.enc_meta[i] for i in ph])
            elif self.ecgemv:
                ix = [self.ec_index[i] for i in ph] if self.ec_index else None
                if len(ph) == 1:
                    cbk.ec_gemv(T[ph[0]], xs[T[ph[0]].cols], y=ys[ph[0]], index=ix and ix[0])
                else:
                    cbk.ec_gemv_group([T[i] for i in ph], xs[T[ph[0]].cols], ys=[ys[i] for i in ph], indexes=ix)
            elif self.ecfmt:
                ix = [self.ec_index[i] for i in ph] if self.ec_index else None
                if len(ph) == 1:
                    cbk.ec_decode_bf16(T[ph[0]], out=ys[ph[0]], index=ix and ix[0])
                else:
                    cbk.ec_decode_group([T[i] for i in ph], outs=[ys[i] for i in ph], indexes=ix)
            elif self.batch == 0 and len(ph) == 1:
                cbk.decode_bf16(T[ph[0]], out=ys[ph[0]])
            elif self.batch == 0:
                cbk.decode_group([T[i] for i in ph], outs=[ys[i] for i in ph])
            elif self.batch > 1 and len(ph) == 1:
                cbk.gemm_small(T[ph[0]], xs[T[ph[0]].cols], Y=ys[ph[0]])
            elif self.batch > 1:
                cbk.gemm_group([T[i] for i in ph], xs[T[ph[0]].cols], Ys=[ys[i] for i in ph])
            elif len(ph) == 1:
                cbk.gemv(T[ph[0]], xs[T[ph[0]].cols], y=ys[ph[0]])
            else:
                cbk.gemv_group([T[i] for i in ph], xs[T[ph[0]].cols], ys=[ys[i] for i in ph])

    def make_chain(self):
        """The step's phases as one GEMV chain (cbk_gemv_chain_*): one persistent launch per step."""
        import fly_decode_amd as cbk
        T, xs, ys = self.tensors, self.xs, self.ys
        self.chain = cbk.GemvChain([([T[i] for i in ph], xs[T[ph[0]].cols], [ys[i] for i in ph])
                                    for ph in self.phases])
        return self.chain

    def run_chain(self):
        self.chain.run()

    def phase_pattern(self):
        """The launches of one layer (the step repeats them), with their algorithmic bytes: a list
        of [tensor names, bytes] (None for workloads of independent single-tensor launches)."""
        if self.name not in STEP_WORKLOADS and not self.name.startswith("mlp_"):
            return None
        per = 4 if self.name in STEP_WORKLOADS else 2
        b, T = max(1, self.batch), self.tensors
        out = []
        for ph in self.phases[:per]:
            nbytes = sum(T[i].compressed_bytes + 4 * b * T[i].rows for i in ph) + 2 * b * T[ph[0]].cols
            out.append(["+".join(self.specs[i][2].name for i in ph), int(nbytes)])
        return out

    def capture(self):
        """The step captured once in a HIP graph (after one eager step)."""
        import torch
        self.step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.step()
        torch.cuda.synchronize()
        return graph

    def algorithmic_bytes(self) -> int:
        """Bytes the method must move per step (the roofline's numerator)."""
        T, b = self.tensors, self.batch
        # with the span index, its byte per 64-bit span is read too
        ix = [((d.total_bits + 63) // 64) if self.ec_index else 0 for d in T] if self.ecfmt else None
        if self.ecgemv:  # the stored entropy-coded form + x read, y written
            return sum(d.stored_bytes + k + 2 * d.cols + 4 * d.rows for d, k in zip(T, ix))
        if self.ecfmt:  # the stored entropy-coded form read + the BF16 written
            return sum(d.stored_bytes + k + 2 * d.n for d, k in zip(T, ix))
        if b == 0:  # decode: compressed reads + the BF16 written; encode: the reverse
            return sum(d.compressed_bytes + 2 * d.n for d in T)
        # packed indices + codebook + Y for every tensor, X once per launch
        return sum(d.compressed_bytes + 4 * b * d.rows for d in T) + \
            sum(2 * b * T[ph[0]].cols for ph in self.phases)

    def kernel_name(self):
        bits = sorted({d.b for d in self.tensors}) if not self.ecfmt else None
        if getattr(self, "chain", None) is not None:
            return f"k_gemv_chain_b{bits[-1]}", f"k_gemv_chain<{bits[-1]}>, one cooperative launch per step"
        if self.encode:
            return "k_enc", "cbk_encode_gpu per tensor (k_enc_clear, k_enc_presence, k_enc_pack)"
        if self.ecfmt:
            k = ("k_ec_gemv" if self.ecgemv else "k_ec_decode") + ("_ix" if self.ec_index else "")
            # the decode's fitted kernel when every block holds at most 8,185 codes
            if not self.ecgemv and all(0 < d.max_block_codes <= 8185 for d in self.tensors):
                k += "_fit"
            return k, k
        if self.batch == 0:
            k = "k_decode_fast"
        elif self.batch == 1:
            k = "k_gemv_rows"
        else:
            k = "k_gemm_valu" if self.batch <= 8 else "k_gemm_mfma"
        grouped = any(len(ph) > 1 for ph in self.phases)
        desc = f"{k}<{bits[-1]}>" + (f" and {k}_group<{bits[-1]}>, every launch of the step" if grouped else "")
        return f"{k}_b{bits[-1]}", desc


# ------------------------------------------------------------------------------------- timing

def time_steps(run_step, steps, stream):
    """Per-step times (ms) from one pair of HIP events per step on the launch stream, plus the
    whole timed region's event time and wall time."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(steps):
        run_step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return per, evs[0].elapsed_time(evs[-1]), wall


def copy_bandwidth(nbytes: int, reps: int = 10):
    """Device-to-device copy of nbytes (read + write counted), median over reps, in GB/s."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        dst.copy_(src)
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * nbytes / float(np.median(times)) / 1e9


def pct(vals, q):
    return float(np.percentile(np.asarray(vals, dtype=np.float64), q))


# ------------------------------------------------------------------------------- CPU baseline

def sample_rows(rows: int, per: int, seed) -> np.ndarray:
    """The first and last row and per - 2 seeded others."""
    rng = np.random.default_rng(seed)
    k = max(0, min(rows, per) - 2)
    mid = rng.choice(np.arange(1, rows - 1), size=k, replace=False) if rows > 2 and k else np.array([], np.int64)
    return np.unique(np.concatenate([[0, rows - 1], mid]).astype(np.int64))


def cpu_baseline(work: Workload, rows_per_tensor: int, seconds: float, threads: int):
    """The oracle (decode + GEMV/GEMM in float64) on sampled rows of every tensor of the workload:
    timed on `threads` host threads and on one, then its results compared with the GPU's output
    of the last timed step.  Returns (cpu_baseline record, check record)."""
    import oracle
    import synth

    oracle.build(force=False)
    X = {}
    for d in work.tensors:
        if d.cols not in X:
            X[d.cols] = synth.workload_x(work.specs[0][0], d.cols, max(1, work.batch))
    # inputs: the sampled rows of every tensor, drawn on the host and encoded by the oracle (not timed)
    t_prep = time.perf_counter()
    jobs = []

    def prep(i):
        cfg, layer, t = work.specs[i]
        rows = sample_rows(t.rows, rows_per_tensor, [cfg, layer, t.tensor_id, 77])
        return i, rows, oracle.encode(synth.workload_rows(cfg, layer, t, rows))

    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        jobs = list(ex.map(prep, range(len(work.specs))))
    prep_s = time.perf_counter() - t_prep

    def run(job):
        i, rows, e = job
        Xi = X[work.tensors[i].cols]
        return oracle.gemm(e, Xi) if work.batch > 1 else oracle.gemv(e, Xi[0])

    def timed(nthreads, budget):
        weights, spent, passes, results = 0, 0.0, 0, None
        while spent < budget and passes < 1000:
            t0 = time.perf_counter()
            if nthreads == 1:
                res = [run(j) for j in jobs]
            else:
                with cf.ThreadPoolExecutor(max_workers=nthreads) as ex:
                    res = list(ex.map(run, jobs))
            spent += time.perf_counter() - t0
            results = results or res
            weights += sum(len(rows) * work.tensors[i].cols for i, rows, _ in jobs)
            passes += 1
        return 2.0 * weights / spent / 1e9, passes, spent, results

    v_all, p_all, s_all, results = timed(threads, seconds)
    v_one, p_one, s_one, _ = timed(1, seconds / 2)

    # the check: the GPU's last timed step against the oracle on the sampled rows
    worst, checked = 0.0, 0
    for (i, rows, _), (ref, absb) in zip(jobs, results):
        y = work.ys[i].float().cpu().numpy().astype(np.float64)
        got = y[rows] if work.batch == 1 else y[:, rows]
        err = np.abs(got - ref)
        ratio = float(np.max(err / np.maximum(TOL * absb, 1e-300))) if err.size else 0.0
        worst = max(worst, ratio)
        checked += got.size
        if not np.all(err <= TOL * absb):
            raise SystemExit(f"output of tensor {i} ({work.specs[i][2].name}, layer {work.specs[i][1]}) "
                             f"differs from the oracle beyond 1e-3 * sum|W x| (worst ratio {ratio:.3g})")
    n_rows = sum(len(rows) for _, rows, _ in jobs)
    record = {
        "value": round(v_all, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "one_thread_value": round(v_one, 4),
        "host_cpus": os.cpu_count(),
        "host_cpus_allowed": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
        "cpu_model": cpu_model(),
        "sample": (f"decode + {'GEMM' if work.batch > 1 else 'GEMV'} (float64) of {n_rows} sampled rows "
                   f"({rows_per_tensor} per tensor, first and last included) of all {len(jobs)} tensors "
                   f"of the step; {p_all} passes in {s_all:.1f} s on {threads} threads, {p_one} passes "
                   f"in {s_one:.1f} s on one thread; drawing and encoding the rows ({prep_s:.1f} s) not "
                   f"timed"),
    }
    check = {"rows": n_rows, "outputs": checked, "tensors": len(jobs),
             "worst_err_over_bound": round(worst, 6), "tolerance": "1e-3 * sum_k |W x|"}
    return record, check


def cpu_baseline_encode(work: Workload, seconds: float):
    """The oracle's encoder (plain C, one host thread) on whole tensors of the workload."""
    import oracle
    import synth

    oracle.build(force=False)
    cfg, layer, t = work.specs[0]
    w = synth.workload_tensor(cfg, layer, t)
    t_total, used = 0.0, 0
    while t_total < seconds and used < 4096:
        t0 = time.perf_counter()
        oracle.encode(w)
        t_total += time.perf_counter() - t0
        used += 1
    return {
        "value": round(2.0 * used * w.size / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"{used} full encodes of one {t.rows}x{t.cols} tensor of the workload with the "
                  f"oracle's encoder (one host thread), {t_total:.1f} s",
    }


def cpu_baseline_decode(work: Workload, seconds: float):
    """The oracle's decoder (plain C, one host thread) on one whole tensor of the workload, encoded
    by the oracle beforehand (not timed)."""
    import oracle
    import synth

    oracle.build(force=False)
    cfg, layer, t = work.specs[0]
    e = oracle.encode(synth.workload_tensor(cfg, layer, t))
    t_total, used = 0.0, 0
    while t_total < seconds and used < 4096:
        t0 = time.perf_counter()
        oracle.decode(e)
        t_total += time.perf_counter() - t0
        used += 1
    return {
        "value": round(2.0 * used * t.rows * t.cols / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"{used} full decodes of one {t.rows}x{t.cols} tensor of the workload with the "
                  f"oracle's decoder (one host thread), {t_total:.1f} s",
    }


def check_decoded(work: Workload, which):
    """The decoded BF16 of tensors `which` after the timed steps against the host weights (exact)."""
    import torch
    import synth
    for i in which:
        cfg, layer, t = work.specs[i]
        got = work.ys[i].view(torch.int16).cpu().numpy().view(np.uint16).reshape(t.rows, t.cols)
        if not np.array_equal(got, synth.workload_tensor(cfg, layer, t)):
            raise SystemExit(f"decode of tensor {i} is not bit-exact")
    return {"tensors": len(which), "bit_exact": True}


def cpu_baseline_ec(work: Workload, seconds: float):
    """The oracle's bit-by-bit decoder of the entropy-coded format (pure Python, one thread) on
    leading rows of one tensor of the workload, growing the sample until about `seconds` pass.
    With the fused GEMV, the oracle's GEMV of those rows (decode, then float64 products)."""
    from oracle import entropy as ec
    import synth

    cfg, layer, t = work.specs[0]
    w = synth.workload_tensor(cfg, layer, t)
    x = synth.workload_x(cfg, t.cols)[0]
    rows, spent, done = 4, 0.0, 0
    while spent < seconds and rows <= t.rows:
        enc = ec.encode(w[:rows])
        t0 = time.perf_counter()
        if work.ecgemv:
            ec.gemv(enc, rows, t.cols, x)
        else:
            ec.decode(enc)
        spent += time.perf_counter() - t0
        done += rows * t.cols
        rows *= 2
    what = "decoder and float64 GEMV" if work.ecgemv else "decoder"
    return {
        "value": round(2.0 * done / spent / 1e9, 6),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"the oracle's bit-by-bit {what} (pure Python, one thread) on the leading 4, 8, ... "
                  f"rows of one {t.rows}x{t.cols} tensor of the workload, {done} weights, {spent:.1f} s",
    }


def check_encoded(work: Workload, which):
    """The device encodings of tensors `which` against the host encoder (exact)."""
    import fly_decode_amd as cbk
    for i in which:
        h = work.tensors[i]
        U, b = (int(v) for v in work.enc_meta[i].cpu().tolist())
        nw = cbk.words_for(work.raws[i].numel(), b)
        ok = (U, b) == (h.U, h.b) and \
            np.array_equal(work.enc_cb[i][:U].cpu().numpy().view(np.uint16), h.codebook) and \
            np.array_equal(work.enc_words[i][:nw].cpu().numpy().view(np.uint32), h.words)
        if not ok:
            raise SystemExit(f"GPU encoding of tensor {i} differs from the host encoder")
    return {"tensors": len(which), "equal_to_host_encoder": True}


def check_ec(work: Workload, which):
    """The entropy-coded outputs of the last timed step for tensors `which`: the decode against
    the host weights (exact); the fused GEMV on 8 sampled rows (first and last included) against the
    C oracle's GEMV of the same weights, within the tolerance.  Returns the record for the line."""
    import torch
    import oracle
    import synth
    oracle.build(force=False)
    worst = 0.0
    for i in which:
        cfg, layer, t = work.specs[i]
        if not work.ecgemv:
            got = work.ys[i].view(torch.int16).cpu().numpy().view(np.uint16).reshape(t.rows, t.cols)
            if not np.array_equal(got, synth.workload_tensor(cfg, layer, t)):
                raise SystemExit(f"entropy-coded decode of tensor {i} is not bit-exact")
            continue
        rows = sample_rows(t.rows, 8, [cfg, layer, t.tensor_id, 99])
        x = synth.workload_x(cfg, t.cols)[0]
        ref, absb = oracle.gemv(oracle.encode(synth.workload_rows(cfg, layer, t, rows)), x)
        got = work.ys[i].cpu().numpy().astype(np.float64)[rows]
        ratio = np.abs(got - ref) / np.maximum(TOL * absb, 1e-300)
        worst = max(worst, float(ratio.max()))
        if not np.all(np.abs(got - ref) <= TOL * absb):
            raise SystemExit(f"entropy-coded GEMV of tensor {i} is outside the tolerance")
    if work.ecgemv:
        return {"tensors": len(which), "rows_per_tensor": 8, "worst_err_over_bound": round(worst, 6),
                "tolerance": "1e-3 * sum_k |W x|"}
    return {"tensors": len(which), "bit_exact": True}


# ------------------------------------------------------------------------- profile summaries

def summarize_trace_main(args):
    """--summarize-trace DIR: the kernel-trace CSV of a rocprofv3 run of this benchmark, reduced to
    the dispatches of its timed steps (the last steps x launches_per_step dispatches of the
    library's kernels), against the JSON line the same run printed."""
    from fly_decode_amd import profiling
    line = json.loads(open(args.line).read().strip().splitlines()[-1])
    profiling.summarize_timed_trace(args.summarize_trace, line, args.out, args.title or line["config"]["workload"],
                                    args.command)
    print(open(args.out).read())


def summarize_counters_main(args):
    from fly_decode_amd import profiling
    profiling.summarize_counters(args.summarize_counters, args.kernel, args.out, args.title, args.command)
    print(open(args.out).read())


def summarize_traffic_main(args):
    from fly_decode_amd import profiling
    fetch, write, cfetch, cwrite = args.summarize_traffic
    rec = profiling.summarize_traffic(args.out, args.kernel, fetch, write, cfetch, cwrite, args.copy_bytes,
                                      args.algorithmic_bytes, args.command,
                                      dispatches_per_unit=args.dispatches_per_unit)
    print(json.dumps(rec, indent=1))


# ------------------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-seconds", type=float, default=0.3,
                    help="after the warm-up steps, keep replaying untimed steps until this much wall "
                         "time has passed (the GPU's clocks rise over the first tens of ms of load)")
    ap.add_argument("--workload", default="l70b_b1", choices=ALL_WORKLOADS)
    ap.add_argument("--tensors", type=int, default=24, help="distinct tensors for the 4096x4096 workloads")
    ap.add_argument("--layers", type=int, default=0,
                    help="layers: the first L of the step workloads (default all), distinct copies for mlp_* (8)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cpu-rows", type=int, default=8, help="sampled rows per tensor for the CPU baseline and check")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU baseline (and with it the check)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of graph replay")
    ap.add_argument("--cap", type=int, default=0, metavar="K",
                    help="lossy: cap every codebook at K entries (cbk_cap_patterns) before encoding")
    ap.add_argument("--no-group", action="store_true", help="one launch per tensor (no grouped phases)")
    ap.add_argument("--ec-index", action="store_true",
                    help="entropy-coded workloads: build the span index at setup and decode with one walk per span")
    ap.add_argument("--tensors-per-call", type=int, default=0, metavar="G",
                    help="the 4096x4096 workloads: tensors per grouped call (default: 4 for decode4096, "
                         "encode4096 and ecdecode4096, 3 for ecgemv4096, 1 for attn4096; 1: one call per tensor)")
    ap.add_argument("--launch", choices=("phases", "chain"), default="phases",
                    help="batch 1: one launch per phase (graph-replayed), or the whole step as one GEMV "
                         "chain (a persistent cooperative launch)")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30, help="size of the in-run copy-bandwidth measurement")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run 3 device-to-device copies of BYTES (counter calibration for the "
                         "traffic figure) and exit")
    ap.add_argument("--summarize-trace", metavar="DIR", help="write a timed-steps kernel summary and exit")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write a traffic record from four --pmc runs and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="write the mean per dispatch of the --pmc runs under DIR... for --kernel and exit")
    ap.add_argument("--line", help="the JSON line the profiled run printed (for --summarize-trace)")
    ap.add_argument("--out", help="output file of a summary")
    ap.add_argument("--title", default="")
    ap.add_argument("--command", default="", help="the command the summarized run executed")
    ap.add_argument("--kernel", default="", help="kernel name prefix (for --summarize-traffic)")
    ap.add_argument("--copy-bytes-calibrated", dest="copy_bytes_cal", type=int, default=0)
    ap.add_argument("--algorithmic-bytes", type=float, default=0.0)
    ap.add_argument("--dispatches-per-unit", type=int, default=1)
    args = ap.parse_args()

    if args.summarize_trace:
        return summarize_trace_main(args)
    if args.summarize_counters:
        return summarize_counters_main(args)
    if args.summarize_traffic:
        args.copy_bytes = args.copy_bytes_cal
        return summarize_traffic_main(args)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (the GEMV would "
              "shard by output rows, each GPU holding a contiguous row slice of every tensor's "
              "stream).", file=sys.stderr)
        sys.exit(2)

    import torch
    import fly_decode_amd as cbk
    from fly_decode_amd import profiling

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        src = torch.ones(args.copy_calibration, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_calibration, "copies": 3}), flush=True)
        return
    cbk.load_library()
    threads = host_threads()
    log(f"workload {args.workload}; host threads {threads} of {os.cpu_count()} CPUs")
    work = Workload(args.workload, count=args.tensors, layers=args.layers, threads=threads, cap=args.cap or None,
                    ec_index=args.ec_index, per_call=args.tensors_per_call)
    if args.no_group:
        work.phases = [[i] for ph in work.phases for i in ph]
    log(f"setup {work.setup_s:.1f} s: {len(work.tensors)} tensors, {len(work.phases)} launches per step, "
        f"{torch.cuda.memory_allocated() / 1e9:.1f} GB allocated on the GPU")

    chain = args.launch == "chain"
    if chain and (work.batch != 1 or work.ecfmt):
        print("--launch chain applies to the batch-1 GEMV workloads", file=sys.stderr)
        sys.exit(2)
    if chain:
        work.make_chain()
        log(f"GEMV chain: {len(work.phases)} phases over {work.chain.grid} workgroups, one launch per step")
    warm0 = time.perf_counter()
    for _ in range(args.warmup):
        work.run_chain() if chain else work.step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    graph = None if (args.no_graph or chain) else work.capture()
    run_step = work.run_chain if chain else graph.replay if graph is not None else work.step
    if graph is not None:
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
    extra = 0
    while time.perf_counter() - warm0 < args.warmup_seconds:
        for _ in range(4):
            run_step()
            extra += 1
        torch.cuda.synchronize()
    if extra:
        log(f"warm-up: {args.warmup} steps + {extra} more to reach {args.warmup_seconds:.2f} s")

    # ---- timed region: K steps, one event pair each
    per_step, region_ms, wall = time_steps(run_step, args.steps, stream)
    ms_step = region_ms / args.steps
    log(f"timed {args.steps} steps: mean {ms_step:.4f} ms/step, median {pct(per_step, 50):.4f} "
        f"(p10 {pct(per_step, 10):.4f}, p90 {pct(per_step, 90):.4f}), wall {wall:.3f} s")
    if chain:
        st = work.chain.check()
        if st != 0:
            print(f"the GEMV chain gave up waiting (status {st})", file=sys.stderr)
            sys.exit(1)
    # outputs of the last timed step, first and last tensor (the GEMV and GEMM workloads are checked
    # on sampled rows of every tensor with the CPU baseline below)
    out_check = None
    if work.encode:
        out_check = check_encoded(work, sorted({0, len(work.raws) - 1}))
        log("device encodings of the first and last tensor equal the host encoder's")
    elif work.ecfmt:
        out_check = check_ec(work, sorted({0, len(work.tensors) - 1}))
        log(f"entropy-coded outputs of the first and last tensor checked: {out_check}")
    elif work.batch == 0:
        out_check = check_decoded(work, sorted({0, len(work.tensors) - 1}))
        log(f"decoded outputs of the first and last tensor checked: {out_check}")

    copy_gbps = copy_bandwidth(args.copy_bytes)
    log(f"device-to-device copy of {args.copy_bytes} B: {copy_gbps:.1f} GB/s (read + write)")

    launches = 1 if chain else len(work.phases)
    step_s = ms_step * 1e-3
    n_total = sum(d.n for d in work.tensors)
    comp_total = work.algorithmic_bytes()
    value = 2.0 * n_total / step_s / 1e9
    comp_gbps = comp_total / step_s / 1e9
    # The step is one graph of back-to-back launches on `stream`, so the step time divided by the
    # launch count is the launches' average duration (inter-launch gaps included, which makes it a
    # slight overestimate; the rocprofv3 summary of the timed steps gives the kernels' own time).
    avg_launch_s = step_s / launches
    algo_per_launch = comp_total / launches
    achieved = algo_per_launch / avg_launch_s / 1e9
    kernel_key, kernel_desc = work.kernel_name()
    # traffic records are per launch, taken on each workload's default launch grouping
    traffic_key = args.workload
    if args.workload in PER_CALL_DEFAULT and work.phases and len(work.phases[0]) != PER_CALL_DEFAULT[args.workload]:
        traffic_key += f"_g{len(work.phases[0])}"
    traffic = profiling.traffic_for(kernel_key, traffic_key)
    bits = sorted({d.b for d in work.tensors}) if not work.ecfmt else [max(max(d.lengths) for d in work.tensors)]

    metric = ("GPU codebook encode of BF16 weights resident in HBM, raw-weight GB/s; % of HBM peak"
              if work.encode else
              "exponent entropy-coded fused GEMV decompressed-weight GB/s at batch 1; % of HBM peak"
              if work.ecgemv else
              "exponent entropy-coded BF16 decode to HBM, decompressed-weight GB/s; % of HBM peak"
              if work.ecfmt else
              "fused codebook-GEMV decompressed-weight GB/s at batch 1; % of HBM peak" if work.batch == 1
              else "standalone codebook decode to BF16 in HBM, decompressed-weight GB/s; % of HBM peak"
              if work.batch == 0 else
              f"fused codebook skinny-GEMM decompressed-weight GB/s at batch {work.batch}; % of HBM peak")
    result = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "tensors": len(work.tensors),
            "shapes": sorted({f"{d.rows}x{d.cols}" for d in work.tensors}),
            "batch": work.batch,
            "layers": work.n_layers,
            ("max_code_bits" if work.ecfmt else "index_bits"): bits,
            "compressed_bytes_per_step": comp_total,
            "raw_bf16_bytes_per_step": 2 * n_total,
            "graph_replay": graph is not None,
            "launch": args.launch if work.batch == 1 and not work.ecfmt else "phases",
            "ec_span_index": bool(work.ec_index) if work.ecfmt else None,
            "tensors_per_launch": max(len(ph) for ph in work.phases),
            "launches_per_step": 2 if chain else 3 * launches if work.encode else 2 * launches if work.ecgemv else launches,
            "codebook_cap": args.cap or None,
            "warmup_seconds_min": args.warmup_seconds,
            "warmup_extra_steps": extra,
            "setup_s": round(work.setup_s, 1),
            "phase_pattern": work.phase_pattern(),
            "weights_generated_on": "gpu" if args.workload in STEP_WORKLOADS and not args.cap else "host",
        },
        "step_ms": {"mean": round(ms_step, 5), "median": round(pct(per_step, 50), 5),
                    "p10": round(pct(per_step, 10), 5), "p90": round(pct(per_step, 90), 5),
                    "min": round(min(per_step), 5), "max": round(max(per_step), 5), "n": len(per_step)},
        "compressed_GBps": round(comp_gbps, 2),
        "pct_hbm_peak": round(100.0 * comp_gbps / HBM_PEAK_GBPS, 2),
        "copy_bw": {"GBps": round(copy_gbps, 1), "bytes": args.copy_bytes,
                    "pct_of_copy_bw": round(100.0 * comp_gbps / copy_gbps, 2),
                    "what": "device-to-device copy in the same run, read + write bytes over its time"},
        "roofline": {
            "bound": "hbm",
            "kernel": kernel_desc,
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": round(traffic["traffic_bytes_per_launch"]) if traffic else None,
            "bytes_per_launch": int(algo_per_launch),
            "avg_launch_us": round(avg_launch_s * 1e6, 3),
            "launches_per_unit": 3 if work.encode else 2 if work.ecgemv else 1,
            "traffic_source": os.path.relpath(profiling.traffic_path(kernel_key, traffic_key), ROOT) if traffic else None,
        },
    }
    if args.workload in STEP_WORKLOADS:
        result["layer_time_us"] = round(ms_step * 1e3 / work.n_layers, 3)
        result["tokens_per_s_equiv"] = round(1.0 / step_s, 2)
    elif not work.encode:
        result["launch_time_us"] = round(avg_launch_s * 1e6, 3)
    if work.batch > 1:
        result["effective_TFLOPs"] = round(2.0 * work.batch * n_total / step_s / 1e12, 3)

    if out_check is not None:
        result["check"] = out_check
    if not args.no_cpu_baseline and work.batch >= 1 and not work.ecgemv:
        log("CPU baseline (oracle on sampled rows of every tensor) and output check ...")
        result["cpu_baseline"], result["check"] = cpu_baseline(work, args.cpu_rows, args.cpu_seconds, threads)
        log(f"check: {result['check']}")
    elif not args.no_cpu_baseline and work.ecfmt:
        log("CPU baseline (oracle entropy decoder) ...")
        result["cpu_baseline"] = cpu_baseline_ec(work, args.cpu_seconds)
    elif not args.no_cpu_baseline and work.encode:
        log("CPU baseline (oracle encoder) ...")
        result["cpu_baseline"] = cpu_baseline_encode(work, args.cpu_seconds)
    elif not args.no_cpu_baseline and work.batch == 0:
        log("CPU baseline (oracle decoder) ...")
        result["cpu_baseline"] = cpu_baseline_decode(work, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
