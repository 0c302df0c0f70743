#!/usr/bin/env python3
"""Benchmark: fused codebook-GEMV decompressed-weight GB/s at batch 1; % of HBM peak.

One step = one pass of the fused decode + GEMV (or skinny GEMM) over every tensor of the workload,
with the compressed tensors already resident in HBM.  Workloads (seeded synthetic BF16 weights,
each tensor with its own codebook):

  attn4096   (default) Llama-7B-shaped 4096x4096 attention projections, N(0, 0.02); 24 distinct
             tensors (654 MB compressed, well above the 256 MB Infinity Cache) so every step reads
             HBM; one cbk_gemv launch per tensor.
  llama7b    full 7B-shaped decode step: 32 layers x {q,k,v,o 4096x4096, gate/up 11008x4096,
             down 4096x11008}, N(0, 0.02) (224 tensors, 10.5 GB).  Per layer four dependent phases:
             [q,k,v] and [gate,up] each one cbk_gemv_group launch (they share their input), o and
             down one cbk_gemv launch each.
  mlp_b8     Llama-7B MLP at batch 8: gate/up 11008x4096 and down 4096x11008, 0.02 * Student-t(4);
             --layers distinct copies (default 8, 1.76 GB); per layer [gate, up] one cbk_gemm_group
             launch (they share X), down one cbk_gemm_small launch.
  l70b_b16   70B-shaped layer at batch 16: q/o 8192x8192, k/v 1024x8192, gate/up 28672x8192,
             down 8192x28672, N(0, 0.015); --layers distinct layers (default 2, 2.8 GB); phases
             grouped as in llama7b (cbk_gemm_group for [q, k, v] and [gate, up]).
  l70b_b1    the same tensors at batch 1, phases grouped as in llama7b.
  decode4096 standalone decode to BF16 in HBM (cbk_decode_bf16) of the attn4096 tensors, one launch
             per tensor; bytes = compressed reads + 2 bytes written per weight.
  ecdecode4096 the attn4096 tensors in the exponent entropy-coded format (sign-mantissa bytes
             raw, exponent Huffman-coded), decoded to BF16 in HBM by cbk_ec_decode_bf16, one launch
             per tensor; bytes = the stored format read + 2 bytes written per weight.
  ecgemv4096 the same entropy-coded tensors, decode fused into the batch-1 GEMV (cbk_ec_gemv: a
             y zero-fill and the fused kernel per tensor); bytes = the stored format + x + y.
  encode4096 the load-time path: cbk_encode_gpu of the attn4096 tensors from raw BF16 already in
             HBM (three launches per tensor); bytes = 2 bytes read per weight + the compressed
             form written; the result of the last step is checked against the host encoder.

The step is captured once in a HIP graph and replayed; the timed region is bracketed by
torch.cuda.synchronize().  Untimed warm-up runs for --warmup steps and at least --warmup-seconds
(0.3 s) of wall time, so that the timed steps see the GPU at its sustained clocks.  `value` = sum over the step of 2*rows*cols (the BF16 bytes the decode
feeds the multiply) / step time.  The dominant kernel's roofline uses its algorithmic bytes per
launch (packed indices ceil(n*b/8) + codebook 2U + X 2*batch*K + Y 4*batch*M) over its average launch
duration, measured with HIP events on the launch stream.  The CPU baseline times the oracle (decode
+ GEMV in float64) on a bounded sample with host threads.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def workload_tensors(name: str, count: int, layers: int):
    """(specs, phases, batch, layer_count): specs are (cfg, layer, tensor) triples; phases are lists
    of spec indices launched together (one launch per phase, phases run in order)."""
    import synth
    if name in ("attn4096", "decode4096", "encode4096", "ecdecode4096", "ecgemv4096"):
        t = synth.WORKLOADS[2][0][0]
        specs = [(2, layer, t) for layer in range(count)]
        return specs, [[i] for i in range(len(specs))], (1 if name in ("attn4096", "ecgemv4096") else 0), len(specs)
    if name in ("llama7b", "l70b_b1", "l70b_b16"):
        cfg = 4 if name == "llama7b" else 5
        tensors, n_layers = synth.WORKLOADS[cfg]
        n_layers = n_layers if name == "llama7b" else layers
        specs, phases = [], []
        for layer in range(n_layers):
            base = len(specs)
            specs += [(cfg, layer, t) for t in tensors]
            names = [t.name for t in tensors]
            for group in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
                phases.append([base + names.index(g) for g in group])
        return specs, phases, (16 if name == "l70b_b16" else 1), n_layers
    if name == "mlp_b8":
        tensors, _ = synth.WORKLOADS[3]
        specs = [(3, layer, t) for layer in range(layers) for t in tensors]
        # per layer: [gate, up] share X (one grouped launch), then down
        return specs, [p for l in range(layers) for p in ([3 * l, 3 * l + 1], [3 * l + 2])], 8, layers
    raise SystemExit(f"unknown workload {name}")


def prepare(specs, threads, raw=False, cap=None):
    """Generate and encode every tensor on the host (threads), upload to the GPU.  With raw=True
    the uploaded form is the BF16 patterns themselves (int16, flat) and the host encodings stay on
    the host, as (raw tensors, host encodings)."""
    import torch
    import synth
    import fly_decode_amd as cbk

    def make(spec):
        cfg, layer, t = spec
        w = synth.workload_tensor(cfg, layer, t)
        return w, cbk.encode(w, cap=cap)

    out, hosts = [], []
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        for i, (w, c) in enumerate(ex.map(make, specs)):
            if raw:
                out.append(torch.from_numpy(w.reshape(-1).view(np.int16)).to("cuda"))
                hosts.append(c)
            else:
                out.append(c.to("cuda"))
            if (i + 1) % 16 == 0 or i + 1 == len(specs):
                log(f"encoded + uploaded {i + 1}/{len(specs)} tensors")
    return (out, hosts) if raw else out


def cpu_baseline(specs, seconds: float, threads: int):
    """The oracle (decode + GEMV, float64) on whole tensors of the workload, rows split over host
    threads, until about `seconds` of wall time have been spent."""
    import oracle
    import synth

    oracle.build(force=False)
    done_w, t_total, used = 0, 0.0, 0
    cfg, layer, t = specs[0]
    w = synth.workload_tensor(cfg, layer, t)
    e = oracle.encode(w)
    x = synth.workload_x(cfg, t.cols)[0]
    y = np.zeros(t.rows, dtype=np.float64)
    ab = np.zeros(t.rows, dtype=np.float64)
    chunk = max(1, t.rows // (threads * 4))
    spans = [(r, min(t.rows, r + chunk)) for r in range(0, t.rows, chunk)]
    while t_total < seconds and used < 4096:
        t0 = time.perf_counter()
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(lambda s: oracle.gemv_rows_into(e, x, s[0], s[1], y, ab), spans))
        t_total += time.perf_counter() - t0
        done_w += t.rows * t.cols
        used += 1
    return {
        "value": round(2.0 * done_w / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{used} full passes of decode+GEMV (float64) over one {t.rows}x{t.cols} tensor "
                  f"of the workload, rows split over {threads} host threads, {t_total:.1f} s",
    }


def cpu_baseline_encode(specs, seconds: float):
    """The oracle's encoder (plain C, one host thread) on whole tensors of the workload, until about
    `seconds` of wall time have been spent."""
    import oracle
    import synth

    oracle.build(force=False)
    cfg, layer, t = specs[0]
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
        "sample": f"{used} full encodes of one {t.rows}x{t.cols} tensor of the workload with the "
                  f"oracle's encoder (one host thread), {t_total:.1f} s",
    }


def cpu_baseline_ec(specs, seconds: float, gemv: bool = False):
    """The oracle's bit-by-bit decoder of the entropy-coded format (pure Python, one thread) on
    leading rows of one tensor of the workload, growing the sample until about `seconds` pass.
    With `gemv`, the oracle's GEMV of those rows (decode, then float64 products) is timed."""
    from oracle import entropy as ec
    import synth

    cfg, layer, t = specs[0]
    w = synth.workload_tensor(cfg, layer, t)
    x = synth.workload_x(cfg, t.cols)[0]
    rows, spent, done = 4, 0.0, 0
    while spent < seconds and rows <= t.rows:
        enc = ec.encode(w[:rows])
        t0 = time.perf_counter()
        if gemv:
            ec.gemv(enc, rows, t.cols, x)
        else:
            ec.decode(enc)
        spent += time.perf_counter() - t0
        done += rows * t.cols
        rows *= 2
    what = "decoder and float64 GEMV" if gemv else "decoder"
    return {
        "value": round(2.0 * done / spent / 1e9, 6),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"the oracle's bit-by-bit {what} (pure Python, one thread) on the leading 4, 8, ... "
                  f"rows of one {t.rows}x{t.cols} tensor of the workload, {done} weights, {spent:.1f} s",
    }


def check_encoded(raws, hosts, codebooks, words, metas, which):
    """The device encodings of tensors `which` against the host encoder (exact)."""
    import fly_decode_amd as cbk
    for i in which:
        h = hosts[i]
        U, b = (int(v) for v in metas[i].cpu().tolist())
        nw = cbk.words_for(raws[i].numel(), b)
        ok = (U, b) == (h.U, h.b) and \
            np.array_equal(codebooks[i][:U].cpu().numpy().view(np.uint16), h.codebook) and \
            np.array_equal(words[i][:nw].cpu().numpy().view(np.uint32), h.words)
        if not ok:
            raise SystemExit(f"GPU encoding of tensor {i} differs from the host encoder")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-seconds", type=float, default=0.3,
                    help="after the warm-up steps, keep replaying untimed steps until this much wall "
                         "time has passed (the GPU's clocks rise over the first tens of ms of load)")
    ap.add_argument("--workload", default="attn4096", choices=["attn4096", "llama7b", "mlp_b8", "l70b_b16", "l70b_b1", "decode4096",
                                                           "encode4096", "ecdecode4096", "ecgemv4096"])
    ap.add_argument("--tensors", type=int, default=24, help="distinct tensors for attn4096")
    ap.add_argument("--layers", type=int, default=0, help="distinct layers for mlp_b8 (8) and l70b_* (2)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of graph replay")
    ap.add_argument("--cap", type=int, default=0, metavar="K",
                    help="lossy: cap every codebook at K entries (cbk_cap_patterns) before encoding")
    ap.add_argument("--no-group", action="store_true", help="one launch per tensor (no grouped phases)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run 3 device-to-device copies of BYTES (counter calibration for the "
                         "traffic figure) and exit")
    args = ap.parse_args()

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
    threads = min(16, os.cpu_count() or 1)
    layers_arg = args.layers or (8 if args.workload == "mlp_b8" else 2)
    specs, phases, batch, n_layers = workload_tensors(args.workload, args.tensors, layers_arg)
    if args.no_group:
        phases = [[i] for ph in phases for i in ph]
    log(f"workload {args.workload}: {len(specs)} tensors, host threads {threads}")
    encode = args.workload == "encode4096"
    ecfmt = args.workload in ("ecdecode4096", "ecgemv4096")
    ecgemv = args.workload == "ecgemv4096"
    t0 = time.perf_counter()
    if ecfmt:
        def make_ec(spec):
            cfg, layer, t = spec
            return cbk.ec_encode(synth.workload_tensor(cfg, layer, t))
        import synth
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            tensors = [e.to("cuda") for e in ex.map(make_ec, specs)]
        log(f"entropy-coded {len(tensors)} tensors")
    elif encode:
        raws, hosts = prepare(specs, threads, raw=True)
        tensors = hosts
        ws = torch.empty(cbk.encode_gpu_workspace_bytes(), dtype=torch.uint8, device="cuda")
        enc_cb = [torch.empty(65536, dtype=torch.int16, device="cuda") for _ in raws]
        enc_words = [torch.empty(cbk.words_for(r.numel(), 16), dtype=torch.int32, device="cuda") for r in raws]
        enc_meta = [torch.zeros(2, dtype=torch.int32, device="cuda") for _ in raws]
    else:
        tensors = prepare(specs, threads, cap=args.cap or None)
    log(f"setup {time.perf_counter() - t0:.1f} s")

    import synth
    xs = {}
    for d in tensors:
        if d.cols not in xs and batch > 0:
            x = synth.workload_x(specs[0][0], d.cols, batch)
            xs[d.cols] = torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16)
    if encode:
        ys = []
    elif batch == 0:  # decode outputs (both formats)
        ys = [torch.empty((d.rows, d.cols), dtype=torch.bfloat16, device="cuda") for d in tensors]
    elif batch == 1:
        xs = {k: v[0] for k, v in xs.items()}
        ys = [torch.empty(d.rows, dtype=torch.float32, device="cuda") for d in tensors]
    else:
        ys = [torch.empty((batch, d.rows), dtype=torch.float32, device="cuda") for d in tensors]

    def step():
        for ph in phases:
            if encode:
                i = ph[0]
                cbk.encode_gpu_launch(raws[i], ws, enc_cb[i], enc_words[i], enc_meta[i])
            elif ecgemv:
                cbk.ec_gemv(tensors[ph[0]], xs[tensors[ph[0]].cols], y=ys[ph[0]])
            elif ecfmt:
                cbk.ec_decode_bf16(tensors[ph[0]], out=ys[ph[0]])
            elif batch == 0:
                cbk.decode_bf16(tensors[ph[0]], out=ys[ph[0]])
            elif batch > 1 and len(ph) == 1:
                cbk.gemm_small(tensors[ph[0]], xs[tensors[ph[0]].cols], Y=ys[ph[0]])
            elif batch > 1:
                cbk.gemm_group([tensors[i] for i in ph], xs[tensors[ph[0]].cols], Ys=[ys[i] for i in ph])
            elif len(ph) == 1:
                cbk.gemv(tensors[ph[0]], xs[tensors[ph[0]].cols], y=ys[ph[0]])
            else:
                cbk.gemv_group([tensors[i] for i in ph], xs[tensors[ph[0]].cols], ys=[ys[i] for i in ph])

    warm0 = time.perf_counter()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
    # Sustained rate: the GPU raises its clocks over the first tens of milliseconds of load (the
    # 70B-shaped layer runs at about 60 % of peak after 5 steps, 67 % after 50, 73 % after 200), so
    # untimed steps continue until --warmup-seconds of wall time have passed since the first one.
    extra = 0
    while time.perf_counter() - warm0 < args.warmup_seconds:
        for _ in range(4):
            if graph is not None:
                graph.replay()
            else:
                step()
            extra += 1
        torch.cuda.synchronize()
    if extra:
        log(f"warm-up: {args.warmup} steps + {extra} more to reach {args.warmup_seconds:.2f} s")

    # ---- timed region: K steps
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    log(f"timed {args.steps} steps: {ms_step:.4f} ms/step (event), wall {wall:.3f} s")
    if encode:
        check_encoded(raws, hosts, enc_cb, enc_words, enc_meta, sorted({0, len(raws) - 1}))
        log("device encodings of the first and last tensor equal the host encoder's")

    # The step is one graph of back-to-back GEMV launches on `stream`, so the event-timed step
    # divided by its launch count is the kernels' average launch duration (inter-kernel gaps
    # included, which makes it a slight overestimate; rocprofv3 kernel traces agree to ~2 %).
    # The encoder is three launches per tensor (clear, presence, pack); its figure below is
    # for the whole encode of one tensor, with the per-kernel split in the rocprofv3 summary.
    launches = len(phases)
    avg_launch_s = ms_step * 1e-3 / launches

    n_total = sum(d.n for d in tensors)
    if ecgemv:  # the stored entropy-coded form + x read, y written
        comp_total = sum(d.stored_bytes + 2 * d.cols + 4 * d.rows for d in tensors)
    elif ecfmt:  # the stored entropy-coded form read + the BF16 written
        comp_total = sum(d.stored_bytes + 2 * d.n for d in tensors)
    elif batch == 0:  # decode: compressed reads + the BF16 written; encode: the reverse
        comp_total = sum(d.compressed_bytes + 2 * d.n for d in tensors)
    else:  # packed indices + codebook + Y for every tensor, X once per launch
        comp_total = sum(d.compressed_bytes + 4 * batch * d.rows for d in tensors) + \
            sum(2 * batch * tensors[ph[0]].cols for ph in phases)
    step_s = ms_step * 1e-3
    value = 2.0 * n_total / step_s / 1e9
    comp_gbps = comp_total / step_s / 1e9
    algo_per_launch = comp_total / launches
    achieved = algo_per_launch / avg_launch_s / 1e9
    bits = sorted({d.b for d in tensors}) if not ecfmt else [max(max(d.lengths) for d in tensors)]
    kernel = ("k_enc" if encode else "k_ec_gemv" if ecgemv else "k_ec_decode" if ecfmt else "k_decode_fast" if batch == 0 else "k_gemv_rows" if batch == 1
              else "k_gemm_valu" if batch <= 8 else "k_gemm_mfma")
    kernel_key = kernel if ecfmt else f"{kernel}_b{bits[-1]}"
    traffic = profiling.traffic_for(kernel_key, args.workload)

    result = {
        "metric": ("GPU codebook encode of BF16 weights resident in HBM, raw-weight GB/s; % of HBM peak"
                   if encode else
                   "exponent entropy-coded fused GEMV decompressed-weight GB/s at batch 1; % of HBM peak"
                   if ecgemv else
                   "exponent entropy-coded BF16 decode to HBM, decompressed-weight GB/s; % of HBM peak"
                   if ecfmt else
                   "fused codebook-GEMV decompressed-weight GB/s at batch 1; % of HBM peak" if batch == 1
                   else "standalone codebook decode to BF16 in HBM, decompressed-weight GB/s; % of HBM peak"
                   if batch == 0 else
                   f"fused codebook skinny-GEMM decompressed-weight GB/s at batch {batch}; % of HBM peak"),
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
            "tensors": len(tensors),
            "shapes": sorted({f"{d.rows}x{d.cols}" for d in tensors}),
            "batch": batch,
            "layers": n_layers,
            ("max_code_bits" if ecfmt else "index_bits"): bits,
            "compressed_bytes_per_step": comp_total,
            "raw_bf16_bytes_per_step": 2 * n_total,
            "graph_replay": graph is not None,
            "launches_per_step": 3 * launches if encode else 2 * launches if ecgemv else launches,
            "codebook_cap": args.cap or None,
            "warmup_seconds_min": args.warmup_seconds,
            "warmup_extra_steps": extra,
        },
        "compressed_GBps": round(comp_gbps, 2),
        "pct_hbm_peak": round(100.0 * comp_gbps / HBM_PEAK_GBPS, 2),
        "layer_time_us": round(ms_step * 1e3 / n_layers, 3),
        "roofline": {
            "bound": "hbm",
            "kernel": ("cbk_encode_gpu per tensor (k_enc_clear, k_enc_presence, k_enc_pack)"
                       if encode else kernel if ecfmt else f"{kernel}<{bits[-1]}>"),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": round(traffic["traffic_bytes_per_launch"]) if traffic else None,
            "bytes_per_launch": int(algo_per_launch),
            "avg_launch_us": round(avg_launch_s * 1e6, 3),
            "launches_per_unit": 3 if encode else 2 if ecgemv else 1,
            "traffic_source": os.path.relpath(profiling.traffic_path(kernel_key, args.workload), ROOT) if traffic else None,
        },
    }
    if not encode:
        result["tokens_per_s_equiv"] = round(1.0 / step_s, 2)
    if batch > 1:
        flops = 2.0 * batch * n_total / step_s
        result["effective_TFLOPs"] = round(flops / 1e12, 3)
    if not args.no_cpu_baseline and batch == 1 and not ecgemv:
        log("CPU baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(specs, args.cpu_seconds, threads)
    elif not args.no_cpu_baseline and ecfmt:
        log("CPU baseline (oracle entropy decoder) ...")
        result["cpu_baseline"] = cpu_baseline_ec(specs, args.cpu_seconds, gemv=ecgemv)
    elif not args.no_cpu_baseline and encode:
        log("CPU baseline (oracle encoder) ...")
        result["cpu_baseline"] = cpu_baseline_encode(specs, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
