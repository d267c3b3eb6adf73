#!/usr/bin/env python3
"""Benchmark of the SSD hot path on one MI355X.

One step = one pass of the whole path over one batch: the chunked prefill of
a Mamba-2 130M-shaped layer (batch 1, 4096 tokens, 24 heads, headdim 64,
d_state 128, 1 group, chunk 256, bf16 operands) through the four prefill
kernels, then one decode token from the prefill's final state through the
decode kernel.  `value` is prefill tokens/s over whole steps.

The decode half of the metric (state-update GB/s against HBM peak) is
measured in the same run on the Codestral-7B decode workload (batch 64,
128 heads, headdim 64, d_state 128, 8 groups, 128 sequential steps, float32
state of 268 MB) and reported under "decode".

The timed steps are launched eagerly (pre-marshalled calls through the C ABI);
the same step replayed from a HIP graph is reported as ms_per_step_graph.
Per-kernel durations come from HIP events around replays of a HIP graph of
20 launches of that kernel alone, on the replay stream.  The
roofline object uses algorithmic bytes / flops per launch (not measured
traffic); "traffic" is HBM bytes per launch from rocprofv3 counters taken
offline for the same command (null when not available).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
TRANSCENDENTAL_PEAK_TPS = 9.83  # v_exp_f32 at a quarter of the fp32 lane rate: 256 x 4 x 16 x 2.4 GHz / 4
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector (packed): 256 CU x 4 SIMD x 16 lanes x 2 x 2 x 2.4 GHz
FP32_PEAK_TFLOPS = 157.3     # MI355X fp32 vector
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-large", action="store_true",
                    help="skip the Mamba-2 2.7B layer prefill measurement")
    ap.add_argument("--no-train", action="store_true",
                    help="skip the training-step (forward + backward) measurement")
    ap.add_argument("--train-only", action="store_true",
                    help="only run --steps forward + backward passes of the 130M layer (for "
                         "profiling) and print their timing")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--copy-calibration", type=int, metavar="MIB", default=0,
                    help="only run a plain device-to-device copy of MIB MiB ten times "
                         "(reference kernel for scaling rocprofv3 byte counters)")
    ap.add_argument("--summarize", metavar="DIR",
                    help="turn rocprofv3 output under DIR into profiles/ summaries and exit")
    return ap.parse_args()


def log(args, msg):
    if not args.quiet:
        print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------ algorithmic work
def cbg_launch(w, T, nseq):
    """Whether the row-split chunk scan reads C.B^T formed in the state-pass
    launch (the library's rule: bf16, P 64, N 128, chunk <= 256, fewer than
    2048 chunk-head units)."""
    nc = (T + nseq * (w.chunk - 1)) // w.chunk
    return (w.dtype == "bf16" and w.P == 64 and w.N == 128 and w.chunk <= 256
            and nc * w.H < 2048)


def prefill_work(w, T, nseq, h0):
    """Algorithmic bytes and flops of the prefill, per kernel (SSD chunked form)."""
    H, P, N, G, Q = w.H, w.P, w.N, w.G, w.chunk
    e = 2 if w.dtype == "bf16" else 4
    state = nseq * H * N * P * 4
    # chunk state (with the chunk-local cumulative decay): x, B, dt read;
    # s = cumsum(dt A) (1 flop per token and head), S = sum_j w_j B_j x_j^T
    # (2 flop per token, n, p)
    k2 = dict(bytes=T * H * P * e + T * G * N * e + T * H * 4 + H * 4,
              flops=T * H + 2 * T * H * N * P)
    # state passing reads h0 and writes h_out (chunk states are implementation overhead)
    k3 = dict(bytes=(state if h0 else 0) + state, flops=2 * (T // Q + nseq) * H * N * P)
    # chunk scan: x, B, C, dt read, y written; C.B^T once per group and chunk (full tile),
    # M.X per head (full tile), C.H_in per head
    cb_bytes, cb_flops = T * G * N * e, T * 2 * Q * N * G
    k4 = dict(bytes=T * H * P * (e + 4) + T * G * N * e + cb_bytes + T * H * 4,
              flops=T * H * (2 * Q * P + 2 * N * P) + cb_flops)
    if cbg_launch(w, T, nseq):  # C.B^T (and the B rows) move to the state-pass launch
        k3 = dict(bytes=k3["bytes"] + cb_bytes, flops=k3["flops"] + cb_flops)
        k4 = dict(bytes=k4["bytes"] - cb_bytes, flops=k4["flops"] - cb_flops)
    return {"chunk_state": k2, "state_pass": k3, "chunk_scan": k4}


def step_work(b, H, P, N, G, e_in):
    """Algorithmic bytes/flops of one decode step: state read+write once."""
    return dict(bytes=2 * b * H * N * P * 4 + b * H * P * (e_in + 4) + 2 * b * G * N * e_in
                + b * H * 4, flops=5 * b * H * N * P)


# ------------------------------------------------------------------- timing
def time_loop(torch, fn, iters):
    """Average ms per call of fn(), with HIP events on the current stream."""
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


def graph_ms(torch, fn, reps, per_graph):
    """Average ms per fn() call, from `reps` replays of a HIP graph holding
    `per_graph` calls (events on the replay stream)."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            fn()
    g.replay()
    torch.cuda.synchronize()
    ms = time_loop(torch, g.replay, reps) / per_graph
    del g
    return ms


def load_traffic():
    """Measured HBM bytes per launch, or {} when absent or taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    if t.get("source_hash") != source_hash():
        return {}
    return {wl: {k: v.get("bytes") for k, v in ks.items()} for wl, ks in t.items()
            if isinstance(ks, dict)}


def roofline(name, work, ms, traffic):
    flops_rate = work["flops"] / (ms * 1e-3) / 1e12
    bytes_rate = work["bytes"] / (ms * 1e-3) / 1e9
    # the bound is the resource whose peak time is larger for this kernel
    t_hbm = work["bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = work["flops"] / (BF16_PEAK_TFLOPS * 1e12)
    tr = traffic.get(name)
    if t_mfma > t_hbm:
        return {"kernel": name, "bound": "mfma", "achieved": round(flops_rate, 2),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(flops_rate / BF16_PEAK_TFLOPS, 4), "traffic": tr,
                "avg_us": round(ms * 1e3, 2)}
    return {"kernel": name, "bound": "hbm", "achieved": round(bytes_rate, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(bytes_rate / HBM_PEAK_GBS, 4),
            "traffic": tr, "avg_us": round(ms * 1e3, 2)}


def cpu_baseline(args, d, w, budget_s=10.0):
    """The fp64 oracle on the whole prefill workload, repeated for about budget_s."""
    import oracle
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    x = d["x"]
    runs = 0
    t0 = time.perf_counter()
    while True:
        oracle.prefill(x, d["dt"], d["A"], d["B"], d["C"], d["D"], None, d["cu_seqlens"],
                       threads=threads)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    T = x.shape[0]
    return {"value": round(runs * T / el, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"whole prefill workload ({T} tokens x {w.H} heads) run {runs} times, "
                      f"fp64 sequential recurrence, {el:.1f} s"}


def copy_calibration(mib):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 10}))


def source_hash():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "state_space_model_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


KERNEL_NAMES = {  # kernel symbol fragment -> bench kernel name (first match wins)
    "k_step_multi": "decode_multi_step", "k_conv1d_step": "conv1d_step",
    "k_gated_rmsnorm": "gated_rmsnorm", "k_s6_summary": "s6_summary", "k_s6_pass": "s6_pass",
    "k_s6_replay": "s6_replay", "k_bwd_scan": "bwd_scan", "k_state_pass_bwd": "state_pass_bwd",
    "k_bwd_ddt": "bwd_ddt", "k_bwd_sums": "bwd_sums", "k_gdn_prep": "gdn_chunk_prep",
    "k_gdn_walk": "gdn_chunk_walk", "k_gdn": "gated_delta_rule",
    "k_chunk_state": "chunk_state", "k_state_pass": "state_pass", "k_chunk_scan": "chunk_scan",
    "k_chunk_map": "chunk_map", "k_step": "decode_step",
}
BWD_SCAN_MODES = {"0": "bwd_scan_dx", "1": "bwd_scan_db", "2": "bwd_scan_dc"}


def _kernel_key(name, grid, train=False):
    for frag, k in KERNEL_NAMES.items():
        if frag in name:
            if k == "bwd_scan":  # template mode: k_bwd_scan<T, MODE, ...>
                mode = name.split(frag, 1)[1].split(",")[1].strip() if "<" in name else ""
                k = BWD_SCAN_MODES.get(mode, k)
            if k == "chunk_state" and "true>" in name:
                k = "chunk_state_bwd"
            if train or k.startswith("bwd") or k.endswith("_bwd"):
                return "mamba2-130m-layer-train", k
            if k == "decode_step":  # the two decode workloads differ in grid size
                return ("codestral-7b-decode-step" if int(grid) > 24 * 256 else
                        "mamba2-130m-layer-prefill"), k
            if k in ("decode_multi_step", "conv1d_step", "gated_rmsnorm"):
                return "codestral-7b-decode-step", k
            if k.startswith("s6_"):
                return "mamba1-w1-selective-scan", k
            if k in ("gated_delta_rule", "gdn_chunk_prep", "gdn_chunk_walk"):
                return "gdn-layer-prefill", k
            return "mamba2-130m-layer-prefill", k
    return None, None


PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d DIR/trace -o run -- "
             "python bench.py --no-cpu-baseline --no-large --no-train --steps 50 --warmup 5 --quiet",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/fetch -o run -- "
             "python bench.py --no-cpu-baseline --no-large --no-train --steps 50 --warmup 5 --quiet",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/write -o run -- "
             "python bench.py --no-cpu-baseline --no-large --no-train --steps 50 --warmup 5 --quiet",
    "mfma": "rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 --output-format csv -d DIR/mfma -o run -- "
            "python bench.py --no-cpu-baseline --no-large --no-train --steps 50 --warmup 5 --quiet",
    "ttrace": "rocprofv3 --kernel-trace --stats --output-format csv -d DIR/ttrace -o run -- "
              "python bench.py --train-only --steps 50 --warmup 5 --quiet",
    "cfetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/cfetch -o run -- "
              "python bench.py --copy-calibration 1024",
    "cwrite": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/cwrite -o run -- "
              "python bench.py --copy-calibration 1024",
}


def summarize(directory):
    """rocprofv3 CSVs -> profiles/*.txt and profiles/traffic.json.

    Expects under DIR: trace/*kernel_stats.csv (kernel trace), fetch/ and write/
    (bench --pmc FETCH_SIZE / WRITE_SIZE), cfetch/ and cwrite/ (the same
    counters over --copy-calibration 1024).
    """
    import glob
    out = {}

    def pmc(sub, counter):
        acc = {}
        for p in glob.glob(os.path.join(directory, sub, "**", "*counter_collection.csv"),
                           recursive=True):
            for r in _read_csv(p):
                if r["Counter_Name"] != counter:
                    continue
                acc.setdefault((r["Kernel_Name"], r["Grid_Size"]), []).append(
                    float(r["Counter_Value"]))
        return acc

    def copy_factor(sub, counter, nbytes):
        vals = [v for (k, g), vs in pmc(sub, counter).items() for v in vs
                if "copy" in k.lower() or "elementwise" in k.lower()]
        big = [v for v in vals if v * 1024 > nbytes / 4]
        if not big:
            return None
        return nbytes / (float(np.median(big)) * 1024)   # true bytes per counted byte

    cal = 1024 << 20
    f_fac = copy_factor("cfetch", "FETCH_SIZE", cal)
    w_fac = copy_factor("cwrite", "WRITE_SIZE", cal)
    traffic = {"source_hash": source_hash(), "fetch_factor": f_fac, "write_factor": w_fac}
    lines = []
    for sub, counter, fac in (("fetch", "FETCH_SIZE", f_fac), ("write", "WRITE_SIZE", w_fac)):
        for (kname, grid), vs in sorted(pmc(sub, counter).items()):
            wl, k = _kernel_key(kname, grid)
            if k is None or fac is None:
                continue
            b = float(np.mean(vs)) * 1024 * fac
            traffic.setdefault(wl, {}).setdefault(k, {})[counter.lower()] = round(b)
            lines.append(f"{wl:28s} {k:14s} {counter:10s} {np.mean(vs):14.1f} KiB/dispatch "
                         f"x {fac:.4f} = {b / 1e6:10.3f} MB ({len(vs)} dispatches)")
    for wl, ks in traffic.items():
        if isinstance(ks, dict):
            for k, v in ks.items():
                if "fetch_size" in v and "write_size" in v:
                    v["bytes"] = v["fetch_size"] + v["write_size"]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(traffic, f, indent=1)
    cmds = "\n".join(f"  {k:7s} {v}" for k, v in PROFILE_COMMANDS.items())
    with open(os.path.join(ROOT, "profiles", "hbm_traffic_counters.txt"), "w") as f:
        f.write("HBM traffic per dispatch from rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by\n"
                "the same counter over a plain 1 GiB device copy (true bytes / counted bytes):\n"
                f"  fetch factor {f_fac}, write factor {w_fac}\n"
                f"kernel sources hash {traffic['source_hash']}\n"
                f"commands (cwd = repository root, DIR = output directory):\n{cmds}\n\n"
                + "\n".join(lines) + "\n")
    mf_util, mf_flops = pmc("mfma", "MfmaUtil"), pmc("mfma", "MfmaFlopsBF16")
    if mf_util:
        from state_space_model_amd import inputs
        w1 = inputs.WORKLOADS[1]
        work = prefill_work(w1, w1.batch * w1.L, w1.batch, h0=False)
        ml = []
        for (kname, grid), vs in sorted(mf_util.items()):
            wl, k = _kernel_key(kname, grid)
            if wl != w1.name or k not in work:
                continue
            issued = float(np.mean(mf_flops.get((kname, grid), [0.0])))
            algo = work[k]["flops"]
            ml.append(f"{k:14s} MfmaUtil {np.mean(vs):6.2f} %   MfmaFlopsBF16 {issued / 1e9:9.3f}"
                      f" GFLOP/dispatch   algorithmic {algo / 1e9:8.3f} GFLOP   issued/algorithmic"
                      f" {issued / algo if algo else 0:5.2f}   ({len(vs)} dispatches)")
        head = ["MFMA utilisation of the prefill kernels on the Mamba-2 130M layer workload",
                "(4096 tokens, 24 heads, P 64, N 128, chunk 256, bf16), rocprofv3 derived",
                "counters: MfmaUtil = sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max(GRBM_GUI_ACTIVE)",
                "x SIMDs) x 100 over each dispatch; MfmaFlopsBF16 = bf16 MFMA flops issued",
                "(padding and masked blocks included), against the algorithmic flops.",
                f"kernel sources hash {traffic['source_hash']}",
                "command (cwd = repository root):", "  " + PROFILE_COMMANDS["mfma"], ""]
        with open(os.path.join(ROOT, "profiles", "mfma_util_prefill130m.txt"), "w") as f:
            f.write("\n".join(head + ml) + "\n")
    tstats = glob.glob(os.path.join(directory, "ttrace", "**", "*kernel_stats.csv"),
                       recursive=True)
    if tstats:
        tl = []
        for r in _read_csv(tstats[0]):
            tl.append(f"{r['Name'][:96]:96s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f}"
                      f" {float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f}"
                      f" {float(r['Percentage']):6.2f}")
        with open(os.path.join(ROOT, "profiles", "kernel_trace_train130m.txt"), "w") as f:
            f.write("rocprofv3 kernel trace of forward + backward of the Mamba-2 130M layer scan\n"
                    "(4096 tokens, 24 heads, P 64, N 128, chunk 256, bf16, h0 = 0, dL/dh_out = 0)\n"
                    f"kernel sources hash {traffic['source_hash']}\n"
                    f"command (cwd = repository root):\n  {PROFILE_COMMANDS['ttrace']}\n\n"
                    f"{'kernel':96s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"
                    f" {'%':>6s}\n" + "\n".join(tl) + "\n")
    stats = glob.glob(os.path.join(directory, "trace", "**", "*kernel_stats.csv"), recursive=True)
    if stats:
        rows = _read_csv(stats[0])
        tl = []
        for r in rows:
            tl.append(f"{r['Name'][:96]:96s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f}"
                      f" {float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f}"
                      f" {float(r['Percentage']):6.2f}")
        with open(os.path.join(ROOT, "profiles", "kernel_trace_prefill130m_decode_codestral.txt"),
                  "w") as f:
            f.write("rocprofv3 kernel trace of the benchmark: prefill of the Mamba-2 130M layer\n"
                    "workload (4096 tokens, 24 heads, P 64, N 128, chunk 256, bf16) + next-token\n"
                    "decode, and the Codestral-7B decode workload (b 64, H 128, G 8, fp32 state).\n"
                    f"kernel sources hash {traffic['source_hash']}\n"
                    f"command (cwd = repository root):\n  {PROFILE_COMMANDS['trace']}\n\n"
                    f"{'kernel':96s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"
                    f" {'%':>6s}\n" + "\n".join(tl) + "\n")
    print(json.dumps(traffic, indent=1))


def prefill_large(args, torch, inputs, ssd, dev):
    """The Mamba-2 2.7B layer prefill (4 x 8192 tokens, 80 heads, h0 given):
    whole-prefill time from HIP-graph replays, tokens/s and the algorithmic
    bytes per second against the HBM peak."""
    wl = inputs.WORKLOADS[2]
    d = inputs.workload_inputs(2)
    T = d["x"].shape[0]
    nseq = len(d["cu_seqlens"]) - 1
    op = torch.bfloat16
    t = lambda a, dt=None: torch.from_numpy(np.ascontiguousarray(a)).to(dev) if dt is None \
        else torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
    run, y, h = ssd.prefill(t(d["x"], op), t(d["dt"]), t(d["A"]), t(d["B"], op), t(d["C"], op),
                            t(d["D"]), t(d["h0"]), chunk=wl.chunk, nseq=nseq, prepare=True)
    run()
    torch.cuda.synchronize()
    ms = graph_ms(torch, run, reps=10, per_graph=2)
    kern = {n: round(graph_ms(torch, lambda st=st: run(st), reps=5, per_graph=2) * 1e3, 2)
            for n, st in (("chunk_state", ssd.STAGE_CHUNK_CUMSUM | ssd.STAGE_CHUNK_STATE),
                          ("state_pass", ssd.STAGE_STATE_PASS),
                          ("chunk_scan", ssd.STAGE_CHUNK_SCAN))}
    work = prefill_work(wl, T, nseq, h0=True)
    # the method's bytes (each input read once, y and h_out written once) and flops
    e = 2
    nbytes = T * (wl.H * wl.P * (e + 4) + 2 * wl.G * wl.N * e + 4 * wl.H) + \
        2 * nseq * wl.H * wl.N * wl.P * 4 + 8 * wl.H
    flops = sum(w["flops"] for w in work.values())
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(args, f"2.7B layer prefill: {ms * 1e3:.1f} us")
    return {"workload": wl.name, "tokens": T, "us": round(ms * 1e3, 2),
            "tokens_per_s": round(T / (ms * 1e-3), 1), "algorithmic_bytes": nbytes,
            "achieved_gb_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "algorithmic_flops": flops,
            "mfma_frac": round(flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4),
            "kernels_us": kern}


def train_work(w, T, nseq):
    """Algorithmic bytes and flops of the backward over the chunked form, for a
    training step (h0 = 0, no dL/dh_out).  Bytes: x, dy, B, C, dt read once;
    dx, ddt, dB, dC written once (float32), dh0 written.  Flops (full tiles, as
    the forward): per group C.B^T (2QN); per head dy.x^T (2QP), the three
    masked products of dX, dB, dC (2QP + 2QN + 2QN), and five state products
    (recomputed chunk state, gradient chunk state and the state terms of dX,
    dB, dC; 2NP each)."""
    H, P, N, G, Q = w.H, w.P, w.N, w.G, w.chunk
    e = 2 if w.dtype == "bf16" else 4
    nbytes = T * (H * P * (2 * e + 4) + G * N * (2 * e + 8) + H * 8) + nseq * H * N * P * 4
    flops = T * (G * 2 * Q * N + H * (4 * Q * P + 4 * Q * N + 10 * N * P))
    return dict(bytes=nbytes, flops=flops)


def training_setup(torch, inputs, ssd, dev, k=1):
    """Prepared forward and backward calls over prefill workload k (bf16; the
    130M layer by default, h0 = 0), with a seeded dL/dy and no dL/dh_out: the
    training forward (which leaves its states for the backward) and the
    backward that takes them; also the backward that recomputes them."""
    wl = inputs.WORKLOADS[k]
    d = inputs.workload_inputs(k)
    T = d["x"].shape[0]
    nseq = len(d["cu_seqlens"]) - 1
    op = torch.bfloat16
    t = lambda a, dt=None: torch.from_numpy(np.ascontiguousarray(a)).to(dev) if dt is None \
        else torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
    dy, _ = inputs.cotangents(T, nseq, wl.H, wl.P, wl.N, 4001, "bf16", dh_out=False)
    args = (t(d["x"], op), t(d["dt"]), t(d["A"]), t(d["B"], op), t(d["C"], op), t(d["D"]))
    h0 = None if d["h0"] is None else t(d["h0"])
    fwd, _, _, saved = ssd.prefill_train(*args, h0, chunk=wl.chunk, nseq=nseq, prepare=True)
    bwd, grads = ssd.prefill_backward(*args, t(dy, op), h0, None, chunk=wl.chunk, nseq=nseq,
                                      saved=saved, prepare=True)
    bwd_re, _ = ssd.prefill_backward(*args, t(dy, op), h0, None, chunk=wl.chunk, nseq=nseq,
                                     prepare=True)
    return wl, T, nseq, fwd, bwd, bwd_re


def training_step_bench(args, torch, inputs, ssd, dev, k=1):
    """Forward + backward of a layer's scan (the pair a training step runs) on
    prefill workload k, each from HIP-graph replays; the backward against its
    algorithmic bytes and flops.  The forward leaves its states for the
    backward; the backward that recomputes them is timed beside it."""
    wl, T, nseq, fwd, bwd, bwd_re = training_setup(torch, inputs, ssd, dev, k)

    def both():
        fwd()
        bwd()

    both()
    torch.cuda.synchronize()
    ms_f = graph_ms(torch, fwd, reps=10, per_graph=10)
    ms_b = graph_ms(torch, bwd, reps=10, per_graph=10)
    ms_fb = graph_ms(torch, both, reps=10, per_graph=10)
    bwd_re()
    torch.cuda.synchronize()
    ms_re = graph_ms(torch, bwd_re, reps=10, per_graph=10)
    wb = train_work(wl, T, nseq)
    tf = wb["flops"] / (ms_b * 1e-3) / 1e12
    gbs = wb["bytes"] / (ms_b * 1e-3) / 1e9
    log(args, f"{wl.name} forward + backward: {ms_fb * 1e3:.1f} us (backward {ms_b * 1e3:.1f})")
    return {"workload": wl.name, "tokens": T, "forward_us": round(ms_f * 1e3, 2),
            "backward_us": round(ms_b * 1e3, 2), "forward_backward_us": round(ms_fb * 1e3, 2),
            "backward_recompute_us": round(ms_re * 1e3, 2),
            "tokens_per_s": round(T / (ms_fb * 1e-3), 1),
            "backward_algorithmic_flops": wb["flops"], "backward_algorithmic_bytes": wb["bytes"],
            "backward_mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "backward_hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def train_only(args):
    """--train-only: `steps` forward + backward passes (for rocprofv3)."""
    import torch
    from state_space_model_amd import inputs, ssd
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    wl, T, nseq, fwd, bwd, _ = training_setup(torch, inputs, ssd, dev)
    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ms = time_loop(torch, lambda: (fwd(), bwd()), args.steps)
    print(json.dumps({"workload": wl.name, "steps": args.steps,
                      "forward_backward_us": round(ms * 1e3, 2)}), flush=True)


def long_context_bench(args, torch, inputs, ssd, dev):
    """The long-context packed batch (8 sequences of 1K-32K tokens, 80 heads,
    each with its own h0, bf16): the whole prefill at every chunk size, from
    HIP-graph replays, against the method's algorithmic bytes."""
    wl = inputs.WORKLOADS[4]
    d = inputs.workload_inputs(4)
    T = d["x"].shape[0]
    nseq = len(d["cu_seqlens"]) - 1
    op = torch.bfloat16
    t = lambda a, dt=None: torch.from_numpy(np.ascontiguousarray(a)).to(dev) if dt is None \
        else torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
    args_ = (t(d["x"], op), t(d["dt"]), t(d["A"]), t(d["B"], op), t(d["C"], op), t(d["D"]),
             t(d["h0"]))
    cu = t(d["cu_seqlens"].astype(np.int32))
    e = 2
    nbytes = T * (wl.H * wl.P * (e + 4) + 2 * wl.G * wl.N * e + 4 * wl.H) + \
        2 * nseq * wl.H * wl.N * wl.P * 4 + 8 * wl.H
    out = {"workload": wl.name, "tokens": T,
           "lengths": [int(v) for v in np.diff(d["cu_seqlens"])], "chunks": {}}
    y = torch.empty((T, wl.H, wl.P), dtype=torch.float32, device=dev)
    h = torch.empty((nseq, wl.H, wl.N, wl.P), dtype=torch.float32, device=dev)
    for q in wl.chunks:
        run, _, _ = ssd.prefill(*args_, chunk=q, cu_seqlens=cu, y=y, h_out=h, prepare=True)
        run()
        torch.cuda.synchronize()
        ms = graph_ms(torch, run, reps=3, per_graph=2)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out["chunks"][str(q)] = {"us": round(ms * 1e3, 1),
                                 "tokens_per_s": round(T / (ms * 1e-3), 1),
                                 "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        del run
        torch.cuda.empty_cache()
    log(args, f"long-context prefill: {out['chunks']}")
    return out


def selective_scan_bench(torch, inputs, ssd, dev):
    """The Mamba-1 selective scan at COREY's W1 shape (batch 1, d_inner 1024,
    L 4096, d_state 16, float16), whole scan from HIP-graph replays."""
    w = inputs.S6_W1
    d = inputs.selective_scan_inputs(w["batch"], w["L"], w["dim"], w["N"], 1100, w["dtype"])
    t = lambda a, o=None: torch.from_numpy(np.ascontiguousarray(a)).to(dev) if o is None \
        else torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(o)
    h16 = torch.float16
    run, y, h = ssd.selective_scan(t(d["x"], h16), t(d["dt"], h16), t(d["A"]), t(d["B"], h16),
                                   t(d["C"], h16), t(d["D"]), None, prepare=True)
    run()
    torch.cuda.synchronize()
    ms = graph_ms(torch, run, reps=10, per_graph=10)
    b, L, dim, N = w["batch"], w["L"], w["dim"], w["N"]
    exps = b * L * dim * N                       # one decay per (token, channel, state)
    nbytes = b * L * dim * (2 + 2 + 4) + 2 * b * L * N * 2 + dim * N * 4 + dim * 4 + b * dim * N * 4
    rate = exps / (ms * 1e-3) / 1e12
    return {"workload": w["name"], "shape": {k: w[k] for k in ("batch", "L", "dim", "N", "dtype")},
            "us": round(ms * 1e3, 2), "tokens_per_s": round(b * L / (ms * 1e-3), 1),
            "achieved_gb_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "roofline": {"bound": "alu", "achieved": round(rate, 3),
                         "peak": TRANSCENDENTAL_PEAK_TPS, "unit": "Texp/s",
                         "frac": round(rate / TRANSCENDENTAL_PEAK_TPS, 4), "traffic": None,
                         "kernel": "selective_scan"}}


def gdn_bench(torch, inputs, ssd, dev):
    """The gated delta rule at its layer shape (batch 1, 4096 tokens, 32 heads
    over 16 query/key groups, K = V = 128, bf16), whole scan from HIP-graph
    replays, in both forms: chunked (chunks of 64 tokens on MFMA; the one the
    binding picks) and token by token.  Per token and head the rule does 6 V K
    flops (S k, the update, S q): that is the algorithmic rate reported; the
    chunked form runs on bf16 MFMA, so its roofline is priced against that
    peak, the streaming form's against the fp32 vector peak."""
    w = inputs.GDN_W
    d = inputs.gdn_inputs([w["L"]] * w["batch"], w["H"], w["G"], w["K"], w["V"], 950,
                          dtype=w["dtype"])
    op = torch.bfloat16
    t = lambda a, o=None: torch.from_numpy(np.ascontiguousarray(a)).to(dev) if o is None \
        else torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(o)
    args = (t(d["q"], op), t(d["k"], op), t(d["v"], op), t(d["g"]), t(d["beta"]), None, None)
    T, H, G, K, V = w["batch"] * w["L"], w["H"], w["G"], w["K"], w["V"]
    flops = 6.0 * T * H * V * K
    us = {}
    for form in ("chunked", "stream"):
        run, o, h = ssd.gated_delta_rule(*args, nseq=w["batch"], form=form, prepare=True)
        run()
        torch.cuda.synchronize()
        us[form] = graph_ms(torch, run, reps=5, per_graph=5) * 1e3
    tf = flops / (us["chunked"] * 1e-6) / 1e12
    tfs = flops / (us["stream"] * 1e-6) / 1e12
    return {"workload": w["name"], "shape": {k: w[k] for k in ("batch", "L", "H", "G", "K", "V",
                                                                 "dtype")},
            "form": "chunked", "us": round(us["chunked"], 2),
            "tokens_per_s": round(T / (us["chunked"] * 1e-6), 1),
            "stream_us": round(us["stream"], 2),
            "stream_ns_per_token_step": round(us["stream"] * 1e3 / w["L"], 2),
            "speedup_vs_stream": round(us["stream"] / us["chunked"], 2),
            "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                         "traffic": None, "kernel": "gdn_chunk_prep+gdn_chunk_walk"},
            "stream_roofline": {"bound": "alu", "achieved": round(tfs, 3),
                                "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                                "frac": round(tfs / FP32_VECTOR_PEAK_TFLOPS, 4),
                                "kernel": "gated_delta_rule"}}


def decode_layer_bench(torch, ssd, w3, dev, ms_scan):
    """One token of the decode layer body (conv1d step + SiLU, the scan, the
    gated RMS norm) at the Codestral shape with synthetic weights."""
    b, H, P, N, G, W = w3.batch, w3.H, w3.P, w3.N, w3.G, 4
    inner, Cn = H * P, H * P + 2 * G * N
    g = torch.Generator(device="cpu").manual_seed(3003)
    r = lambda *s: torch.randn(*s, generator=g)
    xbc = r(b, Cn).to(dev, torch.bfloat16)
    z = r(b, inner).to(dev, torch.bfloat16)
    dt = (torch.rand(b, H, generator=g) * 0.1 + 1e-3).to(dev)
    A = -(torch.rand(H, generator=g) * 15 + 1).to(dev)
    D = torch.rand(H, generator=g).to(dev)
    st = r(b, Cn, W).to(dev)
    cw = (r(Cn, W) / W).to(dev)
    cb = (0.1 * r(Cn)).to(dev)
    h = (0.1 * r(b, H, N, P)).to(dev)
    nw = (torch.rand(inner, generator=g) + 0.5).to(dev)
    run, _ = ssd.decode_layer_step(xbc, z, dt, A, D, st, cw, cb, h, nw, 1e-5, H=H, P=P, N=N, G=G,
                                   prepare=True)
    run()
    torch.cuda.synchronize()
    ms = graph_ms(torch, run, reps=5, per_graph=20)
    return {"shape": {"batch": b, "heads": H, "headdim": P, "d_state": N, "groups": G,
                      "d_conv": W, "conv_channels": Cn, "d_inner": inner, "dtype": "bf16"},
            "us": round(ms * 1e3, 2), "scan_alone_us": round(ms_scan * 1e3, 2),
            "conv_and_norm_us": round((ms - ms_scan) * 1e3, 2)}


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.train_only:
        train_only(args)
        return
    import torch
    from state_space_model_amd import inputs, ssd

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    wl = inputs.WORKLOADS[1]
    d = inputs.workload_inputs(1)
    T = d["x"].shape[0]
    nseq = len(d["cu_seqlens"]) - 1
    op = torch.bfloat16
    t = lambda a, dt=None: torch.from_numpy(np.ascontiguousarray(a)).to(dev) if dt is None \
        else torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
    x, B, C = t(d["x"], op), t(d["B"], op), t(d["C"], op)
    dtt, A, D = t(d["dt"]), t(d["A"]), t(d["D"])
    y = torch.empty((T, wl.H, wl.P), dtype=torch.float32, device=dev)
    h_out = torch.empty((nseq, wl.H, wl.N, wl.P), dtype=torch.float32, device=dev)
    ws = ssd.alloc_workspace(T, nseq, wl.H, wl.P, wl.N, wl.chunk, op, dev)
    # next-token decode inputs (same layer, batch 1)
    rng = np.random.Generator(np.random.PCG64(2001))
    xd = t(inputs.round_bf16(rng.standard_normal((nseq, wl.H, wl.P)).astype(np.float32)), op)
    dtd = t(d["dt"][-1:].copy())
    Bd, Cd = t(d["B"][-1:], op), t(d["C"][-1:], op)
    yd = torch.empty((nseq, wl.H, wl.P), dtype=torch.float32, device=dev)

    run_prefill, _, _ = ssd.prefill(x, dtt, A, B, C, D, None, chunk=wl.chunk, nseq=nseq, y=y,
                                    h_out=h_out, workspace=ws, prepare=True)
    run_decode, _ = ssd.step(xd, dtd, A, Bd, Cd, D, h_out, y=yd, prepare=True)

    def step():
        run_prefill()
        run_decode()

    log(args, f"workload: {wl.name} T={T} H={wl.H} P={wl.P} N={wl.N} Q={wl.chunk}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # ---- the timed region: exactly `steps` whole steps, launched eagerly
    ms_step = time_loop(torch, step, args.steps)
    value = T / (ms_step * 1e-3)
    # the same step replayed from a HIP graph (no host launch cost)
    ms_step_graph = graph_ms(torch, step, reps=max(10, args.steps // 10), per_graph=10)

    # ---- per-kernel durations: each kernel alone, 20 launches per HIP graph
    names = [("chunk_state", ssd.STAGE_CHUNK_CUMSUM | ssd.STAGE_CHUNK_STATE),
             ("state_pass", ssd.STAGE_STATE_PASS), ("chunk_scan", ssd.STAGE_CHUNK_SCAN)]
    kern_ms = {}
    for name, st in names:
        kern_ms[name] = graph_ms(torch, lambda st=st: run_prefill(st), reps=10, per_graph=20)
    kern_ms["decode_step"] = graph_ms(torch, run_decode, reps=10, per_graph=20)
    work = prefill_work(wl, T, nseq, h0=False)
    work["decode_step"] = step_work(nseq, wl.H, wl.P, wl.N, wl.G, 2)
    traffic = load_traffic().get(wl.name, {})
    kernels = [roofline(n, work[n], kern_ms[n], traffic) for n in work]
    dominant = max(kernels, key=lambda k: k["avg_us"])

    # ---- the prefill from HBM: before each repeat a 512 MB buffer is written,
    # which evicts the 256 MB last-level cache (5 untimed + 30 timed repeats)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cold = []
    for i in range(35):
        flush.fill_(i & 0xFF)
        ev0.record()
        run_prefill()
        ev1.record()
        torch.cuda.synchronize()
        if i >= 5:
            cold.append(ev0.elapsed_time(ev1) * 1e3)
    del flush
    cold_us = float(np.median(cold))
    prefill_cold = {"repeats": len(cold), "us_median": round(cold_us, 2),
                    "us_mean": round(float(np.mean(cold)), 2),
                    "us_std": round(float(np.std(cold)), 2),
                    "tokens_per_s": round(T / (cold_us * 1e-6), 1)}

    large = None if args.no_large else prefill_large(args, torch, inputs, ssd, dev)
    longctx = None if args.no_large else long_context_bench(args, torch, inputs, ssd, dev)

    # ---- decode workload (the decode half of the metric)
    w3 = inputs.WORKLOADS[3]
    d3 = inputs.workload_inputs(3)
    S3 = args.decode_steps
    x3, dt3 = t(d3["x"][:S3]), t(d3["dt"][:S3])
    B3, C3 = t(d3["B"][:S3]), t(d3["C"][:S3])
    A3, D3, h3 = t(d3["A"]), t(d3["D"]), t(d3["h"])
    y3 = torch.empty((w3.batch, w3.H, w3.P), dtype=torch.float32, device=dev)

    dec_calls = [ssd.step(x3[s], dt3[s], A3, B3[s], C3[s], D3, h3, y=y3, prepare=True)[0]
                 for s in range(S3)]

    def decode_all():
        for call in dec_calls:
            call()

    decode_all()
    ms_dec = time_loop(torch, decode_all, 3) / S3
    ms_dec_graph = graph_ms(torch, decode_all, reps=3, per_graph=1) / S3
    wd = step_work(w3.batch, w3.H, w3.P, w3.N, w3.G, 4)
    dec_rl = roofline("decode_step", wd, ms_dec, load_traffic().get(w3.name, {}))
    decode = {"workload": w3.name, "steps": S3, "us_per_step": round(ms_dec * 1e3, 2),
              "us_per_step_graph": round(ms_dec_graph * 1e3, 2),
              "state_bytes": w3.batch * w3.H * w3.N * w3.P * 4,
              "gb_per_s": dec_rl["achieved"], "frac_hbm_peak": dec_rl["frac"],
              "tokens_per_s": round(w3.batch / (ms_dec * 1e-3), 1), "roofline": dec_rl}

    # ---- the same 128 steps in one launch (inputs staged for every step): the
    # state crosses HBM once, the update runs at fp32 vector speed
    h3m = t(d3["h"])
    y3m = torch.empty((S3, w3.batch, w3.H, w3.P), dtype=torch.float32, device=dev)
    run_multi, _ = ssd.step_multi(x3, dt3, A3, B3, C3, D3, h3m, y=y3m, prepare=True)
    run_multi()
    torch.cuda.synchronize()
    ms_multi = graph_ms(torch, run_multi, reps=5, per_graph=1)
    elems = w3.batch * w3.H * w3.N * w3.P
    mflops = 5.0 * elems * S3
    mbytes = 2 * elems * 4 + S3 * (w3.batch * w3.H * w3.P * 8 + 2 * w3.batch * w3.G * w3.N * 4 +
                                   w3.batch * w3.H * 4)
    tf = mflops / (ms_multi * 1e-3) / 1e12
    decode_multi = {"workload": w3.name, "steps": S3, "us_total": round(ms_multi * 1e3, 2),
                    "us_per_step": round(ms_multi * 1e3 / S3, 3),
                    "tokens_per_s": round(w3.batch * S3 / (ms_multi * 1e-3), 1),
                    "speedup_vs_single_steps": round(ms_dec_graph * S3 / ms_multi, 2),
                    "roofline": {"bound": "alu", "achieved": round(tf, 2),
                                 "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(tf / FP32_VECTOR_PEAK_TFLOPS, 4),
                                 "traffic": None, "kernel": "step_multi",
                                 "algorithmic_bytes": mbytes}}
    del h3m, y3m

    # ---- the decode layer body around the scan at the same shape (d_conv 4,
    # conv channels H*P + 2*G*N, bf16 activations): conv -> scan -> gated norm
    layer = decode_layer_bench(torch, ssd, w3, dev, ms_dec_graph)

    # ---- Mamba-1 selective scan at the COREY W1 shape (a second scan family)
    s6 = selective_scan_bench(torch, inputs, ssd, dev)

    # ---- the gated delta rule scan (the other scan family)
    gdn = gdn_bench(torch, inputs, ssd, dev)

    # ---- forward + backward of the 130M layer scan (a training step's share)
    train = None if args.no_train else training_step_bench(args, torch, inputs, ssd, dev)
    train_large = None if (args.no_train or args.no_large) else \
        training_step_bench(args, torch, inputs, ssd, dev, k=2)

    # MFMA utilisation estimate of the prefill (algorithmic flops / bf16 peak)
    fl = sum(work[n]["flops"] for n in ("chunk_state", "chunk_scan"))
    mfma_util = fl / (sum(kern_ms[n] for n in kern_ms if n != "decode_step") * 1e-3) / \
        (BF16_PEAK_TFLOPS * 1e12)

    cpu = None if args.no_cpu_baseline else cpu_baseline(args, d, wl)
    out = {
        "metric": "SSD prefill tokens/s + MFMA util; decode state-update GB/s vs HBM peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": nseq, "seq_len": T // nseq, "heads": wl.H,
                   "headdim": wl.P, "d_state": wl.N, "groups": wl.G, "chunk": wl.chunk,
                   "step": "prefill + next-token decode"},
        "roofline": {k: dominant[k] for k in ("bound", "achieved", "peak", "unit", "frac",
                                              "traffic")} | {"kernel": dominant["kernel"]},
        "ms_per_step_graph": round(ms_step_graph, 5),
        "prefill_mfma_util": round(mfma_util, 4),
        "kernels": kernels,
        "prefill_cold_cache": prefill_cold,
        "prefill_2p7b_layer": large,
        "prefill_long_context_varlen": longctx,
        "decode": decode,
        "decode_multi_step": decode_multi,
        "decode_layer_step": layer,
        "selective_scan_w1": s6,
        "gated_delta_rule": gdn,
        "training_step_130m": train,
        "training_step_2p7b": train_large,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
