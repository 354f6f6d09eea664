#!/usr/bin/env python3
"""Benchmark of libgdn's verify window: GDN layer tokens/s and achieved HBM
GB/s at 16 streams x 16-row verify on a 27B-like layer (hk=16, hv=48,
dk=dv=128), every row's state and conv tail recorded.

One step = one gdn_recur_window call over the packed 256 rows, inputs already
resident in HBM.  Prints ONE JSON line (see the keys below).  Extra workloads
(``--workload tree27b`` ...) print the same line for that workload; ``--log``
times the logging pass (gdn_recur_log) instead of the recording one, and its
commit by replay.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--log]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0     # MI355X dense bf16 matrix peak, published
MFMA_FP32_PEAK_TFS = 157.3      # MI355X fp32 matrix peak, published


def window_bytes(shape, n, rows, logged=False):
    """Algorithmic HBM bytes of one window / tree call: every input read once,
    every output written once.  Recorded: every row's state and tail; logged:
    every row's decay, write and key (fp32) instead."""
    C = shape.channels
    S = shape.hv * shape.dk * shape.dv * 4
    if logged:
        per_row_out = (shape.hv + shape.hv * shape.dv + shape.hk * shape.dk) * 4
    else:
        per_row_out = S + 3 * C * 2      # state and tail snapshots
    return (n * S                        # stream states in
            + n * 3 * C * 2              # conv tails in
            + rows * per_row_out         # per-row record or log out
            + rows * C * 2               # packed qkv rows in
            + rows * shape.hv * 2 * 2    # a, b in
            + rows * shape.hv * shape.dv * 4   # o out
            + C * 4 * 4 + 2 * shape.hv * 4)    # conv weights, A_log, dt_bias


def workload_name(name, logged, graph):
    desc = {"verify27b": "16 streams x 16-row verify window",
            "tree27b": "16 streams x 16-node random draft trees",
            "ragged27b": "16 streams, ragged windows U{1..16}",
            "window2b": "1 stream x 16-row verify window on the 2B-like layer"}[name]
    desc += (", per-row decay, write and key logged" if logged else ", per-row state and tail recorded")
    return desc + (" (captured HIP graph replays)" if graph else "")


def replay_bytes(shape, n, path_rows):
    """Algorithmic HBM bytes of one commit by replay: every kept stream's
    state read and written, its path's log entries and raw rows read, its
    tail written (the old tail is read only for paths under three rows and
    is not counted)."""
    C = shape.channels
    S = shape.hv * shape.dk * shape.dv * 4
    per_row = (shape.hv + shape.hv * shape.dv + shape.hk * shape.dk) * 4
    return n * (2 * S + 3 * C * 2) + path_rows * (per_row + C * 2) + 4 * (2 * n + 1)


def prefill_flops(shape, lengths, chunk=64):
    """Algorithmic flops of one chunked prompt pass, counted on the actual
    chunk lengths L (2 flops a multiply-add).  Matrix-core bf16 work inside
    the chunks: K K^T and Q K^T (2 L^2 dk each, per key head), T (beta e^gamma K)
    and T (beta V) (2 L^2 dk, 2 L^2 dv) and P U (2 L^2 dv), per value head.
    fp32 state contractions across chunks, per value head: W M0 and
    (e^gamma Q) M0, which read the state, and (e^{gamma_L - gamma} K)^T U, which
    writes it (2 L dk dv each).  Products an implementation adds (the 0/1-
    selection transposes here) are not counted."""
    dk, dv = shape.dk, shape.dv
    sum_l = sum_l2 = 0
    for n in lengths:
        for c0 in range(0, n, chunk):
            L = min(chunk, n - c0)
            sum_l += L
            sum_l2 += L * L
    bf16 = shape.hk * 2 * (2 * sum_l2 * dk) + shape.hv * (2 * sum_l2 * dk + 2 * 2 * sum_l2 * dv)
    fp32 = shape.hv * 3 * 2 * sum_l * dk * dv
    return bf16, fp32


def measured_traffic(key, source="gdn_rows.hip"):
    """HBM bytes a launch from the committed counter summary, or None when the
    kernel source, or the device header every kernel includes, changed since
    the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    csrc = os.path.join(ROOT, "verify_causal_conv1d_amd", "csrc")
    try:
        rec = json.load(open(path))[key]
        sha = hashlib.sha256(open(os.path.join(csrc, source), "rb").read()).hexdigest()
        sha_h = hashlib.sha256(open(os.path.join(csrc, "gdn_device.h"), "rb").read()).hexdigest()
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != sha or rec.get("device_h_sha256") != sha_h:
        return None
    return int(rec["fetch_bytes"] + rec["write_bytes"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="verify27b",
                    choices=["verify27b", "tree27b", "ragged27b", "window2b", "step", "prefill27b",
                             "inproj_decode27b", "inproj_verify27b", "inproj_prefill27b", "inproj_window2b"])
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a captured HIP graph of the calls (launch-bound workloads)")
    ap.add_argument("--log", action="store_true",
                    help="window workloads: log every row's decay, write and key (gdn_recur_log) "
                         "instead of recording its state and tail; the commit by replay is timed too")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="verify workload: leave out the prompt-pass figures beside the headline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time budget of the oracle baseline sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 256 MiB device copy, a kernel of known traffic "
                         "for scaling hardware byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "libgdn's bench measures one GPU; --gpus must be 1 "
                                   "(the verify path shards by stream or key-head group with no "
                                   "exchange between GPUs)"}))
        sys.exit(2)

    import torch
    from verify_causal_conv1d_amd import gdn
    from verify_causal_conv1d_amd import inputs as gi

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.workload == "prefill27b":
        return bench_prefill(args, torch, gdn, gi, dev)
    if args.workload.startswith("inproj_"):
        return bench_inproj(args, torch, gdn, gi, dev)
    if args.workload == "step":
        return bench_step(args, torch, gdn, gi, dev)

    shape, lengths, kw = gi.workload(args.workload)
    tree = args.workload == "tree27b"
    b = gi.make_batch(shape, lengths, **kw)
    n, R = b.n, b.rows
    params = gdn.LayerParams.from_host(b.params, dev)
    row_start = b.row_start.to(dev)
    qkv, a, bb = b.qkv.to(dev), b.a.to(dev), b.b.to(dev)
    tail, state = b.tail.to(dev), b.state.to(dev)
    parent = b.parent.to(dev) if tree else None
    out = torch.empty((R, shape.hv, shape.dv), dtype=torch.float32, device=dev)
    max_rows = max(lengths)
    if args.log:
        la = torch.empty((R, shape.hv), dtype=torch.float32, device=dev)
        ld = torch.empty((R, shape.hv, shape.dv), dtype=torch.float32, device=dev)
        lk = torch.empty((R, shape.hk, shape.dk), dtype=torch.float32, device=dev)
    else:
        tsnap = torch.empty((R, 3, shape.channels), dtype=torch.bfloat16, device=dev)
        ssnap = torch.empty((R, shape.hv, shape.dk, shape.dv), dtype=torch.float32, device=dev)

    def step():
        if args.log:
            gdn.recur_log(shape, params, row_start, qkv, a, bb, tail, state, out, la, ld, lk,
                          max_rows=max_rows, parent=parent)
        elif tree:
            gdn.recur_tree(shape, params, row_start, parent, qkv, a, bb, tail, state, out, tsnap,
                           ssnap, max_rows=max_rows)
        else:
            gdn.recur_window(shape, params, row_start, qkv, a, bb, tail, state, out, tsnap, ssnap,
                             max_rows=max_rows)

    if args.copy_calibration:
        copy_calibration(torch, dev)

    if args.graph:
        step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        step = graph.replay

    # the timed region (events on the launch stream, torch's current stream,
    # which is the stream libgdn launches on), then per-launch events
    wall, avg_ms, med_ms = timed(torch, dev, step, args.steps, args.warmup)

    cold_ms = cold_timed(torch, dev, step) if not args.graph else None
    bytes_per_launch = window_bytes(shape, n, R, logged=args.log)
    achieved_gbs = bytes_per_launch / (avg_ms * 1e-3) / 1e9
    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = R * args.steps / wall

    replay = None
    if args.log:
        # each stream keeps its last row (chains) or its drawn leaf (trees),
        # replayed onto copies of the states: a commit's kernel time, alone
        if tree:
            acc = b.accept
        else:
            acc = b.row_start[1:] - 1
        acc_d = acc.to(dtype=torch.int32, device=dev)
        path_rows = sum(len(gi.path_to_root(b.parent[int(b.row_start[s]):int(b.row_start[s + 1])].tolist(),
                                            int(acc[s]) - int(b.row_start[s])))
                        for s in range(n))
        tail_c, state_c = tail.clone(), state.clone()

        def commit():
            gdn.commit_replay(shape, row_start, acc_d, qkv, la, ld, lk, tail_c, state_c,
                              max_rows=max_rows, parent=parent)

        _, c_avg, c_med = timed(torch, dev, commit, args.steps, args.warmup)
        rb = replay_bytes(shape, n, path_rows)
        replay = {"kernel": "replay_kernel", "ms_avg": round(c_avg, 5), "ms_median": round(c_med, 5),
                  "algorithmic_bytes": rb, "hbm_gbs": round(rb / (c_avg * 1e-3) / 1e9, 1)}

    prefill_obj = None
    if args.workload == "verify27b" and not args.log and not args.graph and not args.no_prefill:
        # the prompt pass on the same layer (four packed prompts, T = 8,306),
        # beside the headline: event-timed passes back to back, run while the
        # GPU is still busy (before the CPU baseline leaves it idle)
        pb, p_wall, p_avg, p_med, _, p_roof = prefill_pass(torch, gdn, gi, dev, 30, 10, cold=False)
        prefill_obj = {
            "workload": "4 prompts of 512, 1024, 2048 and 4722 rows packed in one pass, chunk 64",
            "tokens_per_s": round(pb.rows * 30 / p_wall, 1),
            "pass_ms_avg": round(p_avg, 5), "pass_ms_median": round(p_med, 5),
            "roofline": p_roof,
            "kernel_split": "profiles/prefill27b_kernel_trace.md",
        }

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(b, tree, args.cpu_seconds, logged=args.log)

    # the instantiation that runs: dk = 128, logged or recording
    row_kernel = (f"rows_kernel<{shape.dk}, {'true' if args.log else 'false'}, "
                  f"{'true' if tree and not args.log else 'false'}>")
    line = {
        "metric": "GDN layer tokens/s and achieved HBM GB/s at 16 streams x 16-row verify",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (bf16 inputs)",
        "data": "synthetic",
        "config": {
            "workload": workload_name(args.workload, args.log, args.graph),
            "layer": {"hk": shape.hk, "hv": shape.hv, "dk": shape.dk, "dv": shape.dv, "conv_width": 4},
            "streams": n, "rows": R, "seed": kw["seed"],
        },
        "hbm_gbs": round(achieved_gbs, 1),
        "kernel_ms_avg": round(avg_ms, 5),
        "kernel_ms_median": round(med_ms, 5),
        "kernel_ms_cold_median": None if cold_ms is None else round(cold_ms, 5),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(f"{row_kernel}/{args.workload}" + ("_log" if args.log else "")),
            "kernel": row_kernel,
            "algorithmic_bytes_per_launch": bytes_per_launch,
        },
        "cpu_baseline": cpu,
    }
    if replay is not None:
        line["commit_by_replay"] = replay
    if prefill_obj is not None:
        line["prefill"] = prefill_obj
    print(json.dumps(line), flush=True)


def bench_step(args, torch, gdn, gi, dev):
    """One-row decode steps on the small layer (1 stream): latency-bound, so
    the figure is microseconds a step, eager and from captured graph replays
    (64 steps a graph); the roofline line gives the algorithmic bytes and the
    time they would take at the HBM peak."""
    shape, lengths, kw = gi.workload("step")
    b = gi.make_batch(shape, lengths, **kw)
    params = gdn.LayerParams.from_host(b.params, dev)
    qkv, a, bb = b.qkv.to(dev), b.a.to(dev), b.b.to(dev)
    tail, state = b.tail.to(dev), b.state.to(dev)
    out = torch.empty((1, shape.hv, shape.dv), dtype=torch.float32, device=dev)

    def one():
        gdn.conv_step(shape, params, qkv, a, bb, tail, state, out)

    per_graph = 64
    one()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            one()
    wall_e, avg_e, med_e = timed(torch, dev, one, args.steps, args.warmup)
    wall_g, avg_g, med_g = timed(torch, dev, graph.replay, max(1, args.steps // 8), 2)
    us_graph = med_g * 1e3 / per_graph
    nbytes = window_bytes(shape, 1, 1)   # one row: its state and tail written back instead of recorded
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(b, False, min(args.cpu_seconds, 3.0))
    line = {
        "metric": "GDN one-row decode step latency",
        "value": round(med_e * 1e3, 3), "unit": "us",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall_e * 1e3 / args.steps, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 (bf16 inputs)", "data": "synthetic",
        "config": {"workload": "1 stream, one-row step, state and tail updated in place",
                   "layer": {"hk": shape.hk, "hv": shape.hv, "dk": shape.dk, "dv": shape.dv, "conv_width": 4},
                   "seed": kw["seed"]},
        "eager_us_median": round(med_e * 1e3, 3), "graph_us_per_step": round(us_graph, 3),
        "graph_steps_per_s": round(1e6 / us_graph, 1),
        "roofline": {"bound": "latency", "algorithmic_bytes_per_step": nbytes,
                     "ideal_us_at_hbm_peak": round(nbytes / (HBM_PEAK_GBS * 1e3), 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def copy_calibration(torch, dev):
    """One plain 256 MiB device copy (256 MiB read, 256 MiB written), whose
    counter readings scale the kernels' byte counters."""
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def cold_timed(torch, dev, step, calls=10):
    """Median event time of single calls, each after a 512 MB scratch write
    that evicts the 256 MB last-level cache (the write is outside the events)."""
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    ms = []
    for _ in range(calls):
        scratch.fill_(1)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        step()
        e.record(stream)
        torch.cuda.synchronize()
        ms.append(s.elapsed_time(e))
    del scratch
    ms.sort()
    return ms[len(ms) // 2]


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def timed(torch, dev, step, steps, warmup):
    """Warm-up, then the timed region: ``steps`` launches back to back,
    bracketed by synchronisations, the wall clock and one event pair on
    torch's current stream (where libgdn launches).  Returns the wall seconds,
    the event time a launch (the average launch duration, inter-launch gaps
    included) and the median of a second, untimed pass with an event pair
    around each launch (per-launch event records add several microseconds of
    gap each, so they stay out of the timed region)."""
    for _ in range(warmup):
        step()
    stream = torch.cuda.current_stream(dev)
    first, last = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    first.record(stream)
    for _ in range(steps):
        step()
    last.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_ms = first.elapsed_time(last) / steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return wall, avg_ms, ms[len(ms) // 2]


PREFILL_KERNELS = "qk_kernel, intra_kernel, sweep_kernel"


def prefill_pass(torch, gdn, gi, dev, steps, warmup, copy_cal=False, cold=True):
    """Timed chunked prompt passes over the four packed prompts: (batch,
    wall seconds, event-timed average and median ms, cold median ms or None,
    the roofline object)."""
    shape, lengths, kw = gi.workload("prefill27b")
    b = gi.make_batch(shape, lengths, **kw)
    params = gdn.LayerParams.from_host(b.params, dev)
    seq_start = b.row_start.to(dev)
    qkv, a, bb = b.qkv.to(dev), b.a.to(dev), b.b.to(dev)
    tail, state = b.tail.to(dev), b.state.to(dev)
    out = torch.empty((b.rows, shape.hv, shape.dv), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.prefill_workspace_bytes(shape, b.n, b.rows), dtype=torch.uint8, device=dev)

    def step():
        gdn.prefill_chunked(shape, params, seq_start, qkv, a, bb, tail, state, out, ws,
                            max_len=max(lengths))

    if copy_cal:
        copy_calibration(torch, dev)
    wall, avg_ms, med_ms = timed(torch, dev, step, steps, warmup)
    cold_ms = cold_timed(torch, dev, step) if cold else None
    f_bf16, f_fp32 = prefill_flops(shape, lengths)
    ideal_s = f_bf16 / (MFMA_BF16_PEAK_TFS * 1e12) + f_fp32 / (MFMA_FP32_PEAK_TFS * 1e12)
    fp32_equiv = f_fp32 + f_bf16 * MFMA_FP32_PEAK_TFS / MFMA_BF16_PEAK_TFS
    roof = {
        "bound": "mfma", "achieved": round(fp32_equiv / (avg_ms * 1e-3) / 1e12, 2), "peak": MFMA_FP32_PEAK_TFS,
        "unit": "TFLOP/s", "frac": round(ideal_s / (avg_ms * 1e-3), 4),
        "traffic": measured_traffic("prefill27b", "gdn_prefill.hip"),
        "kernel": f"whole pass ({PREFILL_KERNELS})",
        "flops_bf16": f_bf16, "flops_fp32": f_fp32,
        "note": "achieved counts bf16 flops at the fp32/bf16 peak ratio; frac = ideal time "
                "(bf16 flops at 2.5 PF + fp32 flops at 157.3 TF) over the measured pass; the fp32 "
                "state contractions run as exact three-term bf16 products on the bf16 matrix cores",
    }
    return b, wall, avg_ms, med_ms, cold_ms, roof


def bench_prefill(args, torch, gdn, gi, dev):
    """One step = one chunked prompt pass over the four packed prompts."""
    shape, lengths, kw = gi.workload("prefill27b")
    b, wall, avg_ms, med_ms, cold_ms, roof = prefill_pass(torch, gdn, gi, dev, args.steps, args.warmup,
                                                           copy_cal=args.copy_calibration)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_prefill(b, args.cpu_seconds)
    line = {
        "metric": "GDN layer prefill tokens/s (chunked prompt pass)",
        "value": round(b.rows * args.steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 matrix operands, f32 state", "data": "synthetic",
        "config": {"workload": "4 prompts of 512, 1024, 2048 and 4722 rows packed in one pass, chunk 64",
                   "layer": {"hk": shape.hk, "hv": shape.hv, "dk": shape.dk, "dv": shape.dv,
                             "conv_width": 4},
                   "prompts": lengths, "rows": b.rows, "seed": kw["seed"]},
        "pass_ms_avg": round(avg_ms, 5), "pass_ms_median": round(med_ms, 5),
        "pass_ms_cold_median": round(cold_ms, 5),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def inproj_work(shape, rows, hidden, group):
    """Algorithmic bytes and bf16 matrix flops of one in-projection call: x in,
    packed codes and bf16 scales and biases in, qkv, a, b out (bf16); two
    flops a weight and row."""
    n = shape.channels + 2 * shape.hv
    nbytes = rows * hidden * 2 + n * hidden // 2 + n * (hidden // group) * 4 + rows * n * 2
    return nbytes, 2 * rows * n * hidden


def inproj_kernel_name(torch, dev, shape, rows, hidden, group):
    """The kernel instantiation gdn_inproj_affine4 launches for ``rows`` (the
    library picks it by tile count against the compute units), which names
    its measured traffic."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    features = shape.channels + 2 * shape.hv
    if rows <= 32:
        blocks = (features + 15) // 16
        j = (hidden // 128 + 7) // 8
        nfd = next((c for c in (3, 2) if 4 * ((blocks + c - 1) // c) >= 3 * cus), 1)
        if rows <= 16 and j <= 5 and 4 * nfd * (hidden // group) <= 512 * 3:
            return f"inproj_decode_kernel<{nfd}, {j}>"
        return f"inproj_small_kernel<{1 if rows <= 16 else 2}, {2 if blocks // 2 >= cus else 1}>"
    ft = (features + 127) // 128
    if ft * ((rows + 127) // 128) <= cus:
        return "inproj_large_kernel<2, 2>"
    return "inproj_large_kernel<1, 4>" if rows > 512 else "inproj_large_kernel<1, 2>"


def bench_inproj(args, torch, gdn, gi, dev):
    """One step = one gdn_inproj_affine4 call (hidden rows -> qkv, a, b)."""
    shape, rows, hidden, group, seed = gi.inproj_workload(args.workload)
    t = gi.make_inproj(shape, rows, hidden, group, seed)
    x = t.x.to(dev)
    # the weights are repacked once, as at load time (not timed)
    wq, sc, bi = gdn.inproj_pack(shape, t.wq.to(dev), t.scales.to(dev), t.biases.to(dev), group)
    qkv = torch.empty((rows, shape.channels), dtype=torch.bfloat16, device=dev)
    a = torch.empty((rows, shape.hv), dtype=torch.bfloat16, device=dev)
    b = torch.empty((rows, shape.hv), dtype=torch.bfloat16, device=dev)

    def step():
        gdn.inproj_affine4(shape, x, wq, sc, bi, qkv, a, b, group)

    if args.copy_calibration:
        copy_calibration(torch, dev)
    wall, avg_ms, med_ms = timed(torch, dev, step, args.steps, args.warmup)
    cold_ms = cold_timed(torch, dev, step)
    nbytes, flops = inproj_work(shape, rows, hidden, group)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_BF16_PEAK_TFS * 1e12)
    kernel = inproj_kernel_name(torch, dev, shape, rows, hidden, group)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(nbytes / (avg_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(t_hbm / (avg_ms * 1e-3), 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(flops / (avg_ms * 1e-3) / 1e12, 2),
                "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s", "frac": round(t_mfma / (avg_ms * 1e-3), 4)}
    roof.update({"traffic": measured_traffic(f"{kernel}/{args.workload}", "gdn_inproj.hip"), "kernel": kernel,
                 "algorithmic_bytes_per_launch": nbytes, "flops_bf16_per_launch": flops})
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_inproj(t, args.cpu_seconds)
    line = {
        "metric": "GDN in-projection rows/s (affine 4-bit weights -> qkv, a, b)",
        "value": round(rows * args.steps / wall, 1),
        "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 (4-bit affine weights, fp32 accumulation)", "data": "synthetic",
        "config": {"workload": f"{rows} rows of hidden {hidden} -> qkv, a, b of the "
                               f"{'27B' if shape.hv == 48 else '2B'}-like layer, group {group}",
                   "rows": rows, "hidden": hidden, "features": shape.channels + 2 * shape.hv,
                   "group": group, "seed": seed},
        "kernel_ms_avg": round(avg_ms, 5), "kernel_ms_median": round(med_ms, 5),
        "kernel_ms_cold_median": None if cold_ms is None else round(cold_ms, 5),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_inproj(t, budget_s):
    """The oracle's fp64 projection on a bounded sample: the first 1, 2, 4, ...
    rows of the same call, until about budget_s seconds."""
    import oracle
    from verify_causal_conv1d_amd import inputs as gi
    xb = gi.bf16_bits(t.x)
    wq, sb, bb = t.wq.numpy(), gi.bf16_bits(t.scales), gi.bf16_bits(t.biases)
    rows, el, n = 0, 0.0, 1
    while el < budget_s and n <= t.rows:
        t0 = time.perf_counter()
        oracle.inproj.project(xb[:n], wq, sb, bb, t.group)
        el += time.perf_counter() - t0
        rows += n
        n *= 2
    try:   # the BLAS threads numpy's product ran on
        from threadpoolctl import threadpool_info
        cores = max(i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas")
    except (ImportError, ValueError):
        cores = 1
    return {"value": round(rows / el, 2), "unit": "rows/s", "cores": cores, "cpu": cpu_model(),
            "kind": "oracle", "sample": f"the first 1, 2, 4, ... rows of the call ({rows} rows in all, "
                                        f"weights dequantised each time), numpy fp64, {el:.1f} s wall"}


def cpu_baseline_prefill(b, budget_s):
    """The oracle's recurrent prompt pass on a bounded sample: the first
    ``n`` rows of the 512-row prompt, grown until about budget_s seconds."""
    import numpy as np
    import oracle
    from verify_causal_conv1d_amd import inputs as gi
    h = dict(conv_w=b.params.conv_w.numpy(), a_log=b.params.a_log.numpy(),
             dt_bias=b.params.dt_bias.numpy(), qkv=gi.bf16_bits(b.qkv), a=gi.bf16_bits(b.a),
             b=gi.bf16_bits(b.b), tail=gi.bf16_bits(b.tail), state=b.state.numpy().astype(np.float64))
    rows, el = 0, 0.0
    n = 64
    while el < budget_s and n <= b.rows:
        ss = np.array([0, n], np.int32)
        t0 = time.perf_counter()
        oracle.prefill(b.shape, h["conv_w"], h["a_log"], h["dt_bias"], ss, h["qkv"][:n], h["a"][:n],
                       h["b"][:n], h["tail"][:1], h["state"][:1])
        el += time.perf_counter() - t0
        rows += n
        n *= 2
    return {"value": round(rows / el, 2), "unit": "tokens/s", "cores": oracle.max_threads(), "cpu": cpu_model(),
            "kind": "oracle", "sample": f"recurrent prompt passes of 64, 128, ... rows ({rows} rows in all), "
                                        f"fp64, {el:.1f} s wall"}


def cpu_baseline(b, tree, budget_s, logged=False):
    """The fp64 oracle, as it stands, on the same inputs: whole calls repeated
    until about ``budget_s`` seconds of wall time have passed (recording every
    row's state, or logging every row, as the timed GPU call does)."""
    import numpy as np
    import oracle
    from verify_causal_conv1d_amd import inputs as gi
    h = dict(conv_w=b.params.conv_w.numpy(), a_log=b.params.a_log.numpy(),
             dt_bias=b.params.dt_bias.numpy(), row_start=b.row_start.numpy(),
             qkv=gi.bf16_bits(b.qkv), a=gi.bf16_bits(b.a), b=gi.bf16_bits(b.b),
             tail=gi.bf16_bits(b.tail), state=b.state.numpy().astype(np.float64))
    calls = 0
    t0 = time.perf_counter()
    while True:
        kw = dict(snap64=False, snap32=not logged, tail_snap=not logged, log=logged)
        if tree:
            oracle.tree(b.shape, h["conv_w"], h["a_log"], h["dt_bias"], h["row_start"],
                        b.parent.numpy(), h["qkv"], h["a"], h["b"], h["tail"], h["state"], **kw)
        else:
            oracle.window(b.shape, h["conv_w"], h["a_log"], h["dt_bias"], h["row_start"],
                          h["qkv"], h["a"], h["b"], h["tail"], h["state"], **kw)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or calls >= 10000:
            break
    return {"value": round(b.rows * calls / el, 2), "unit": "tokens/s", "cores": oracle.max_threads(), "cpu": cpu_model(),
            "kind": "oracle",
            "sample": f"{calls} whole calls of the same workload ({b.rows} rows each), fp64, "
                      f"{el:.1f} s wall"}


if __name__ == "__main__":
    main()
