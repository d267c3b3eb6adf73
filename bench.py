#!/usr/bin/env python3
"""Benchmark of the SSD hot path on one MI355X.

One step = one pass of the whole hot path over one batch: the chunked
prefill of a Mamba-2 2.7B-shaped layer (4 sequences of 8192 tokens, 80
heads, headdim 64, d_state 128, 1 group, chunk 256, bf16 operands, an
initial state per sequence) through the prefill kernels, then one decode
token for the 4 sequences from the prefill's final states through the
decode kernel.  `value` is prefill tokens/s over whole steps, the inputs
resident in device memory.  Before its W warm-up steps the step runs for
--preheat seconds (1.5 by default; the count is reported), so that the K
timed steps see the clocks the GPU holds under sustained load rather than
the swing that follows idle time.  Inside the timed region every kernel of the step
is bracketed by HIP events on the stream it runs on, which gives each
kernel's average duration; the roofline object is the longest one's
algorithmic bytes (or flops) per launch over that duration.  After timing, the
outputs of the last timed step (y, the decode output and the advanced state)
are compared with the fp64 oracle on every element ("parity"), and the same
oracle run, timed on the host, is the CPU baseline.

Other workloads of the same run, reported under their own keys: the Mamba-2
130M layer prefill (`prefill_130m_layer`), the long-context packed batch at
every chunk size (`prefill_long_context_varlen`), the Codestral-7B decode
(`decode`, `decode_multi_step`, `decode_layer_step`), the Mamba-1 selective
scan, the gated delta rule and forward + backward training steps.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--preheat S]
       [--sections a,b,...] [--no-cpu-baseline] [--no-parity]
"""
import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
TRANSCENDENTAL_PEAK_TPS = 9.83  # v_exp_f32 at a quarter of the fp32 lane rate: 256 x 4 x 16 x 2.4 GHz / 4
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector (packed): 256 CU x 4 SIMD x 16 lanes x 2 x 2 x 2.4 GHz
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
SECTIONS = ("headline", "small", "longctx", "decode", "s6", "gdn", "train")
PARITY_TOL = 2e-2            # max-abs on y and the state, bf16 operands
SSM_REL_TOL = 1e-2           # max|dy| / max|y_ref - D x|


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--preheat", type=float, default=1.5, metavar="SECONDS",
                    help="run the headline step for this long before its warm-up steps, so "
                         "that the timed steps see the GPU's sustained-load clocks")
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--sections", default=",".join(SECTIONS),
                    help="comma-separated subset of " + ",".join(SECTIONS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the oracle check of the timed outputs (profiling runs)")
    ap.add_argument("--train-only", action="store_true",
                    help="only run --steps forward + backward passes of the 130M layer (for "
                         "profiling) and print their timing")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--copy-calibration", type=int, metavar="MIB", default=0,
                    help="only run a plain device-to-device copy of MIB MiB ten times "
                         "(reference kernel for scaling rocprofv3 byte counters)")
    ap.add_argument("--summarize", metavar="DIR",
                    help="turn rocprofv3 output under DIR into profiles/ summaries and exit")
    a = ap.parse_args()
    a.sections = [s for s in a.sections.split(",") if s]
    bad = [s for s in a.sections if s not in SECTIONS]
    if bad:
        ap.error(f"unknown sections {bad}")
    return a


def log(args, msg):
    if not args.quiet:
        print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------ algorithmic work
def cbg_launch(w, T, nseq):
    """Whether the row-split chunk scan runs and reads C.B^T formed in the
    state-pass launch (the library's rule: bf16, P 64, N 128, chunk <= 256,
    fewer than 2048 chunk-head units)."""
    nc = (T + nseq * (w.chunk - 1)) // w.chunk
    return (w.dtype == "bf16" and w.P == 64 and w.N == 128 and w.chunk <= 256
            and nc * w.H < 2048)


def prefill_totals(w, T, nseq, h0):
    """The method's algorithmic work for the whole prefill (per token:
    bytes H P (e + 4) + 2 G N e + 4 H, flops 2 Q N G + H (2 Q P + 4 N P); plus
    the states h0 (if given) and h_out)."""
    H, P, N, G, Q = w.H, w.P, w.N, w.G, w.chunk
    e = 2 if w.dtype == "bf16" else 4
    state = nseq * H * N * P * 4
    nbytes = T * (H * P * (e + 4) + 2 * G * N * e + 4 * H) + (state if h0 else 0) + state + 8 * H
    flops = T * (2 * Q * N * G + H * (2 * Q * P + 4 * N * P))
    return dict(bytes=nbytes, flops=flops)


def prefill_work(w, T, nseq, h0, plan=None):
    """Algorithmic bytes and flops of each prefill launch: what the launch must
    read and write of the method's tensors, and the contraction flops it must
    do (chunk-state round trips are implementation overhead, not counted).
    x is read by two launches (the chunk states and the output), so the
    per-launch bytes sum to more than the whole prefill's.  With the state
    walk (plan["state"] == "walk") stages 1, 2 and 4 are one launch group,
    "state_walk" (the B-fragment copy, the walk and its fix-up)."""
    H, P, N, G, Q = w.H, w.P, w.N, w.G, w.chunk
    e = 2 if w.dtype == "bf16" else 4
    state = nseq * H * N * P * 4
    # chunk state (with the chunk-local cumulative decay): x, B, dt read;
    # s = cumsum(dt A) (1 flop per token and head), S = sum_j w_j B_j x_j^T
    # (2 flop per token, n, p)
    k2 = dict(bytes=T * H * P * e + T * G * N * e + T * H * 4 + H * 4,
              flops=T * H + 2 * T * H * N * P)
    # state passing reads h0 and writes h_out
    k3 = dict(bytes=(state if h0 else 0) + state, flops=2 * (T // Q + nseq) * H * N * P)
    # chunk scan: x, B, C, dt read, y written; C.B^T once per group and chunk
    # (full tile), M.X per head (full tile), C.H_in per head
    cb_bytes, cb_flops = T * G * N * e, T * 2 * Q * N * G
    k4 = dict(bytes=T * H * P * (e + 4) + T * G * N * e + cb_bytes + T * H * 4,
              flops=T * H * (2 * Q * P + 2 * N * P) + cb_flops)
    row_cbg = plan["scan"] == "rows" if plan else cbg_launch(w, T, nseq)
    if row_cbg and w.dtype == "bf16" and P == 64 and N == 128 and Q <= 256:
        # C.B^T (and the B rows) move to the state-pass launch
        k3 = dict(bytes=k3["bytes"] + cb_bytes, flops=k3["flops"] + cb_flops)
        k4 = dict(bytes=k4["bytes"] - cb_bytes, flops=k4["flops"] - cb_flops)
    if plan and plan["state"] == "walk":
        return {"state_walk": dict(bytes=k2["bytes"] + k3["bytes"], flops=k2["flops"] + k3["flops"]),
                "chunk_scan": k4}
    return {"chunk_state": k2, "state_pass": k3, "chunk_scan": k4}


def stage_parts(ssd, plan):
    """The launch groups of a prefill, as (name, stage bits) in order."""
    if plan["state"] == "walk":
        return [("state_walk", ssd.STAGE_CHUNK_CUMSUM | ssd.STAGE_CHUNK_STATE | ssd.STAGE_STATE_PASS),
                ("chunk_scan", ssd.STAGE_CHUNK_SCAN)]
    return [("chunk_state", ssd.STAGE_CHUNK_CUMSUM | ssd.STAGE_CHUNK_STATE),
            ("state_pass", ssd.STAGE_STATE_PASS), ("chunk_scan", ssd.STAGE_CHUNK_SCAN)]


def step_work(b, H, P, N, G, e_in):
    """Algorithmic bytes/flops of one decode step: state read+write once."""
    return dict(bytes=2 * b * H * N * P * 4 + b * H * P * (e_in + 4) + 2 * b * G * N * e_in
                + b * H * 4, flops=5 * b * H * N * P)


# ------------------------------------------------------------------- timing
def time_loop(torch, fn, iters):
    """Average ms per call of fn(), with HIP events on the current stream."""
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()  # recorded once beforehand, as in timed_steps
    e.record()
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
    # the first graph timed in a process replays about 10 % slower than later
    # ones of the same launches (measured: 545, then 502, 497, 494 us a step at
    # the 2.7B layer): one is captured, timed and dropped first; and each is
    # replayed for 0.2 s before it is timed (capture leaves the GPU idle, and
    # the clocks swing for a few ms after idle time)
    for _ in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                fn()
        t_end = time.perf_counter() + 0.2
        while time.perf_counter() < t_end:
            for _ in range(4):
                g.replay()
            torch.cuda.synchronize()
        ms = time_loop(torch, g.replay, reps) / per_graph
        del g
    return ms


def timed_steps(torch, parts, steps):
    """Run `steps` steps of the launches in `parts` ((name, fn) in order) on the
    current stream, an event recorded before the first launch and after each
    one (the event that ends a step also starts the next).  Returns (ms per
    whole step, {name: average ms of that launch})."""
    n = len(parts)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps * n + 1)]
    # each event recorded once before the timed region: a first record costs
    # the host more than later ones, which would leave gaps between launches
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    evs[0].record()
    for k in range(steps):
        for i, (_, fn) in enumerate(parts):
            fn()
            evs[k * n + i + 1].record()
    torch.cuda.synchronize()
    total = evs[0].elapsed_time(evs[-1]) / steps
    per = {name: sum(evs[k * n + i].elapsed_time(evs[k * n + i + 1]) for k in range(steps)) / steps
           for i, (name, _) in enumerate(parts)}
    return total, per


# the profiled kernels of each launch group the bench times as one part
GROUP_KERNELS = {"state_walk": ("b_frag", "state_walk", "walk_fixup")}


def group_traffic(traffic):
    """Per-kernel HBM bytes -> per launch group: a group's bytes are the sum of
    its kernels' (None when one of them was not profiled)."""
    out = dict(traffic)
    for group, ks in GROUP_KERNELS.items():
        if group in traffic:
            vals = [traffic.get(k) for k in ks]
            out[group] = None if any(v is None for v in vals) else sum(vals)
    return out


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


# ---------------------------------------------------------------- host facts
def source_hash():
    """Hash of the kernel sources (what the profiles were taken on)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "state_space_model_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def tree_hash():
    """Hash of everything the measurement depends on: kernel sources, the C
    header and this file."""
    import hashlib
    h = hashlib.sha256(source_hash().encode())
    for p in (os.path.join(ROOT, "include", "ssd.h"), os.path.abspath(__file__)):
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def git_head():
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                           text=True, timeout=10)
        return r.stdout.strip() or None if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        return None


def rocm_version():
    try:
        with open("/opt/rocm/.info/version") as f:
            return f.read().strip()
    except OSError:
        return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def provenance(torch):
    return {"git_head": git_head(), "tree_sha16": tree_hash(), "kernel_sources_sha16": source_hash(),
            "rocm": rocm_version(), "torch": torch.__version__, "hip": torch.version.hip,
            "device": torch.cuda.get_device_name(0)}


def to_dev(torch, dev, a, dt=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return t if dt is None else t.to(dt)


def maxabs(a, b, block=1 << 22):
    fa, fb = np.asarray(a).reshape(-1), np.asarray(b).reshape(-1)
    assert fa.size == fb.size
    m = 0.0
    for i in range(0, fa.size, block):
        d = np.abs(fa[i:i + block].astype(np.float64) - fb[i:i + block].astype(np.float64))
        m = max(m, float(np.max(d, initial=0.0)))
    return m


# ------------------------------------------------------- the headline step
def headline(args, torch, inputs, ssd, dev):
    """The 2.7B-layer prefill + next-token decode step (the `value`).  Builds and
    uploads the inputs now and returns the function that warms up and times the
    step, so that other GPU work can run in between (a GPU that has been idle
    runs its first ~50 ms of load at lower clocks: without it the first timed
    steps run about 8 % slower)."""
    wl = inputs.WORKLOADS[2]
    d = inputs.workload_inputs(2)
    T = d["x"].shape[0]
    nseq = len(d["cu_seqlens"]) - 1
    op = torch.bfloat16
    t = lambda a, dt=None: to_dev(torch, dev, a, dt)
    x, B, C = t(d["x"], op), t(d["B"], op), t(d["C"], op)
    dtt, A, D, h0 = t(d["dt"]), t(d["A"]), t(d["D"]), t(d["h0"])
    y = torch.empty((T, wl.H, wl.P), dtype=torch.float32, device=dev)
    h_out = torch.empty((nseq, wl.H, wl.N, wl.P), dtype=torch.float32, device=dev)
    ws = ssd.alloc_workspace(T, nseq, wl.H, wl.P, wl.N, wl.G, wl.chunk, op, dev)
    # next-token decode inputs for the 4 sequences (same layer)
    rng = np.random.Generator(np.random.PCG64(2002))
    xd_h = inputs.round_bf16(rng.standard_normal((nseq, wl.H, wl.P)).astype(np.float32))
    cu = d["cu_seqlens"]
    last = cu[1:] - 1
    dtd_h, Bd_h, Cd_h = d["dt"][last].copy(), d["B"][last].copy(), d["C"][last].copy()
    xd, dtd, Bd, Cd = t(xd_h, op), t(dtd_h), t(Bd_h, op), t(Cd_h, op)
    yd = torch.empty((nseq, wl.H, wl.P), dtype=torch.float32, device=dev)

    run_prefill, _, _ = ssd.prefill(x, dtt, A, B, C, D, h0, chunk=wl.chunk, nseq=nseq, y=y,
                                    h_out=h_out, workspace=ws, prepare=True)
    run_decode, _ = ssd.step(xd, dtd, A, Bd, Cd, D, h_out, y=yd, prepare=True)
    plan = ssd.plan(T, nseq, wl.H, wl.P, wl.N, wl.G, wl.chunk, op)
    stages = stage_parts(ssd, plan)
    parts = [(n, (lambda st=st: run_prefill(st))) for n, st in stages] + \
        [("decode_step", run_decode)]

    # the device buffers, released once the step has been timed
    bufs = [x, B, C, y, h_out, ws, dtt, xd, dtd, Bd, Cd, yd]
    del x, B, C, ws

    def go():
        def step():
            run_prefill()
            run_decode()

        log(args, f"headline: {wl.name} T={T} nseq={nseq} H={wl.H} P={wl.P} N={wl.N} Q={wl.chunk}")
        # sustained load first: from idle, and for a few ms after other work,
        # the clocks swing (the chunk scan takes 290 -> 360 -> 285 us over the
        # first ~40 steps) before settling
        pre, t_end = 0, time.perf_counter() + args.preheat
        while time.perf_counter() < t_end:
            for _ in range(8):
                step()
            torch.cuda.synchronize()
            pre += 8
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        # ---- the timed region: exactly `steps` whole steps, each launch bracketed by events
        ms_step, kern_ms = timed_steps(torch, parts, args.steps)
        ms_prefill = sum(kern_ms[n] for n, _ in stages)
        value = T / (ms_step * 1e-3)
        # the same step replayed from a HIP graph (no host launch cost), before
        # the host copies below leave the GPU idle; every step computes the
        # same outputs from the same inputs, so the replays leave them as the
        # timed steps did
        ms_step_graph = graph_ms(torch, step, reps=5, per_graph=2)
        # outputs of the last step, for the parity check below
        y_h = y.cpu().numpy()
        yd_h, h_h = yd.cpu().numpy(), h_out.cpu().numpy()

        work = prefill_work(wl, T, nseq, h0=True, plan=plan)
        work["decode_step"] = step_work(nseq, wl.H, wl.P, wl.N, wl.G, 2)
        traffic = group_traffic(load_traffic().get(wl.name, {}))
        kernels = [roofline(n, work[n], kern_ms[n], traffic) for n in work]
        dominant = max(kernels, key=lambda k: k["avg_us"])
        tot = prefill_totals(wl, T, nseq, h0=True)
        prefill = {"us": round(ms_prefill * 1e3, 2), "tokens_per_s": round(T / (ms_prefill * 1e-3), 1),
                   "algorithmic_bytes": tot["bytes"], "algorithmic_flops": tot["flops"],
                   "hbm_frac": round(tot["bytes"] / (ms_prefill * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                   "mfma_frac": round(tot["flops"] / (ms_prefill * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4)}
        bufs.clear()
        torch.cuda.empty_cache()

        parity = cpu = None
        if not args.no_parity or not args.no_cpu_baseline:
            parity, cpu = check_and_baseline(args, d, wl, (xd_h, dtd_h, Bd_h, Cd_h), y_h, yd_h, h_h)
        config = {"workload": wl.name, "batch": nseq, "seq_len": T // nseq, "heads": wl.H,
                  "headdim": wl.P, "d_state": wl.N, "groups": wl.G, "chunk": wl.chunk,
                  "h0": "given", "step": "prefill + next-token decode of every sequence"}
        config["kernels"] = plan
        preheat = {"seconds": args.preheat, "steps": pre}
        return dict(value=value, ms_step=ms_step, ms_step_graph=ms_step_graph, config=config,
                    preheat=preheat,
                    dominant=dominant, kernels=kernels, prefill=prefill, parity=parity, cpu=cpu)

    return go


def check_and_baseline(args, d, wl, dec, y, yd, h):
    """The fp64 oracle on the step's inputs: every element of the prefill
    output, the decode output and the advanced state against the GPU's, and
    the oracle's own time (all cores: the whole workload; one thread: a sample
    of heads) as the CPU baseline."""
    import oracle
    T = d["x"].shape[0]
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    ry, rh = oracle.prefill(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"],
                            d["h0"].astype(np.float64), d["cu_seqlens"], threads=threads)
    el = time.perf_counter() - t0
    parity = None
    if not args.no_parity:
        xd, dtd, Bd, Cd = dec
        ryd = oracle.step(xd, dtd, d["A"], Bd, Cd, d["D"], rh, threads=threads)  # rh advances
        ey, eyd, eh = maxabs(y, ry), maxabs(yd, ryd), maxabs(h, rh)
        ssm = 0.0
        for i in range(0, T, 8192):
            ssm = max(ssm, float(np.max(np.abs(
                ry[i:i + 8192] - d["D"][None, :, None].astype(np.float64) * d["x"][i:i + 8192]))))
        ok = max(ey, eyd, eh) <= PARITY_TOL and ey <= SSM_REL_TOL * ssm
        parity = {"y_max_abs": float(f"{ey:.4g}"), "decode_y_max_abs": float(f"{eyd:.4g}"),
                  "state_max_abs": float(f"{eh:.4g}"),
                  "y_over_ssm_scale": float(f"{ey / ssm:.4g}"), "tol": PARITY_TOL,
                  "ssm_rel_tol": SSM_REL_TOL, "elements": int(y.size + yd.size + h.size),
                  "ok": bool(ok)}
        log(args, f"parity: {parity}")
    del ry, rh
    cpu = None
    if not args.no_cpu_baseline:
        hs = 8  # one-thread sample: 8 of the heads, every token
        dsel = dict(x=np.ascontiguousarray(d["x"][:, :hs]), dt=np.ascontiguousarray(d["dt"][:, :hs]),
                    A=d["A"][:hs], D=d["D"][:hs],
                    h0=np.ascontiguousarray(d["h0"][:, :hs]).astype(np.float64))
        t1 = time.perf_counter()
        oracle.prefill(dsel["x"], dsel["dt"], dsel["A"], d["B"], d["C"], dsel["D"], dsel["h0"],
                       d["cu_seqlens"], threads=1)
        el1 = time.perf_counter() - t1
        one = T * hs / wl.H / el1
        cpu = {"value": round(T / el, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"the whole workload ({T} tokens x {wl.H} heads, h0 given) once, "
                         f"fp64 sequential recurrence, {el:.2f} s on {threads} threads",
               "single_thread": {"value": round(one, 1), "unit": "tokens/s",
                                 "sample": f"{hs} of the {wl.H} heads, every token, "
                                           f"{el1:.2f} s; scaled to all heads"},
               "cpu_model": cpu_model()}
        log(args, f"cpu baseline: {cpu}")
    return parity, cpu


# ------------------------------------------------- the 130M layer prefill
def small_layer(args, torch, inputs, ssd, dev):
    """The Mamba-2 130M layer prefill (4096 tokens, 24 heads) + next-token
    decode: whole step, each launch, and the prefill from HBM (the last-level
    cache overwritten before each repeat)."""
    wl = inputs.WORKLOADS[1]
    d = inputs.workload_inputs(1)
    T = d["x"].shape[0]
    nseq = len(d["cu_seqlens"]) - 1
    op = torch.bfloat16
    t = lambda a, dt=None: to_dev(torch, dev, a, dt)
    x, B, C = t(d["x"], op), t(d["B"], op), t(d["C"], op)
    dtt, A, D = t(d["dt"]), t(d["A"]), t(d["D"])
    y = torch.empty((T, wl.H, wl.P), dtype=torch.float32, device=dev)
    h_out = torch.empty((nseq, wl.H, wl.N, wl.P), dtype=torch.float32, device=dev)
    ws = ssd.alloc_workspace(T, nseq, wl.H, wl.P, wl.N, wl.G, wl.chunk, op, dev)
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

    for _ in range(args.warmup):
        step()
    ms_step = time_loop(torch, step, max(args.steps, 50))
    ms_graph = graph_ms(torch, step, reps=20, per_graph=10)
    plan = ssd.plan(T, nseq, wl.H, wl.P, wl.N, wl.G, wl.chunk, op)
    kern_ms = {n: graph_ms(torch, lambda st=st: run_prefill(st), reps=10, per_graph=20)
               for n, st in stage_parts(ssd, plan)}
    kern_ms["decode_step"] = graph_ms(torch, run_decode, reps=10, per_graph=20)
    work = prefill_work(wl, T, nseq, h0=False, plan=plan)
    work["decode_step"] = step_work(nseq, wl.H, wl.P, wl.N, wl.G, 2)
    traffic = group_traffic(load_traffic().get(wl.name, {}))
    kernels = [roofline(n, work[n], kern_ms[n], traffic) for n in work]
    # the prefill from HBM: before each repeat a 512 MB buffer is written,
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
    tot = prefill_totals(wl, T, nseq, h0=False)
    log(args, f"130M layer step {ms_step * 1e3:.1f} us, prefill from HBM {cold_us:.1f} us")
    return {"workload": wl.name, "tokens": T, "kernels_used": plan,
            "us_per_step": round(ms_step * 1e3, 2),
            "us_per_step_graph": round(ms_graph * 1e3, 2),
            "tokens_per_s": round(T / (ms_step * 1e-3), 1), "kernels": kernels,
            "prefill_cold_cache": {"repeats": len(cold), "us_median": round(cold_us, 2),
                                   "us_mean": round(float(np.mean(cold)), 2),
                                   "us_std": round(float(np.std(cold)), 2),
                                   "tokens_per_s": round(T / (cold_us * 1e-6), 1),
                                   "hbm_frac": round(tot["bytes"] / (cold_us * 1e-6) /
                                                     (HBM_PEAK_GBS * 1e9), 4),
                                   "mfma_frac": round(tot["flops"] / (cold_us * 1e-6) /
                                                      (BF16_PEAK_TFLOPS * 1e12), 4)}}


def long_context_bench(args, torch, inputs, ssd, dev):
    """The long-context packed batch (8 sequences of 1K-32K tokens, 80 heads,
    each with its own h0, bf16): the whole prefill at every chunk size, from
    HIP-graph replays, against the method's algorithmic bytes and flops."""
    wl = inputs.WORKLOADS[4]
    d = inputs.workload_inputs(4)
    T = d["x"].shape[0]
    nseq = len(d["cu_seqlens"]) - 1
    op = torch.bfloat16
    t = lambda a, dt=None: to_dev(torch, dev, a, dt)
    args_ = (t(d["x"], op), t(d["dt"]), t(d["A"]), t(d["B"], op), t(d["C"], op), t(d["D"]),
             t(d["h0"]))
    cu = t(d["cu_seqlens"].astype(np.int32))
    out = {"workload": wl.name, "tokens": T,
           "lengths": [int(v) for v in np.diff(d["cu_seqlens"])], "chunks": {}}
    y = torch.empty((T, wl.H, wl.P), dtype=torch.float32, device=dev)
    h = torch.empty((nseq, wl.H, wl.N, wl.P), dtype=torch.float32, device=dev)
    from dataclasses import replace
    for q in wl.chunks:
        run, _, _ = ssd.prefill(*args_, chunk=q, cu_seqlens=cu, y=y, h_out=h, prepare=True)
        run()
        torch.cuda.synchronize()
        ms = graph_ms(torch, run, reps=3, per_graph=2)
        tot = prefill_totals(replace(wl, chunk=q), T, nseq, h0=True)
        out["chunks"][str(q)] = {"us": round(ms * 1e3, 1),
                                 "tokens_per_s": round(T / (ms * 1e-3), 1),
                                 "hbm_frac": round(tot["bytes"] / (ms * 1e-3) /
                                                   (HBM_PEAK_GBS * 1e9), 4),
                                 "mfma_frac": round(tot["flops"] / (ms * 1e-3) /
                                                    (BF16_PEAK_TFLOPS * 1e12), 4)}
        del run
        torch.cuda.empty_cache()
    log(args, f"long-context prefill: {out['chunks']}")
    return out


def decode_bench(args, torch, inputs, ssd, dev):
    """The Codestral-7B decode workload: 128 single steps (the decode half of
    the metric), the same steps in one launch, and the decode layer body."""
    w3 = inputs.WORKLOADS[3]
    d3 = inputs.workload_inputs(3)
    S3 = args.decode_steps
    t = lambda a: to_dev(torch, dev, a)
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
    # the same steps in one launch (inputs staged for every step): the state
    # crosses HBM once, the update runs at fp32 vector speed
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
    multi = {"workload": w3.name, "steps": S3, "us_total": round(ms_multi * 1e3, 2),
             "us_per_step": round(ms_multi * 1e3 / S3, 3),
             "tokens_per_s": round(w3.batch * S3 / (ms_multi * 1e-3), 1),
             "speedup_vs_single_steps": round(ms_dec_graph * S3 / ms_multi, 2),
             "roofline": {"bound": "alu", "achieved": round(tf, 2),
                          "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(tf / FP32_VECTOR_PEAK_TFLOPS, 4),
                          "traffic": None, "kernel": "step_multi", "algorithmic_bytes": mbytes}}
    del h3m, y3m
    layer = decode_layer_bench(torch, ssd, w3, dev, ms_dec_graph)
    log(args, f"decode: {ms_dec * 1e3:.1f} us per step ({decode['frac_hbm_peak']:.3f} of HBM)")
    return decode, multi, layer


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


def selective_scan_bench(torch, inputs, ssd, dev):
    """The Mamba-1 selective scan at COREY's W1 shape (batch 1, d_inner 1024,
    L 4096, d_state 16, float16), whole scan from HIP-graph replays."""
    w = inputs.S6_W1
    d = inputs.selective_scan_inputs(w["batch"], w["L"], w["dim"], w["N"], 1100, w["dtype"])
    t = lambda a, o=None: to_dev(torch, dev, a, o)
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
    t = lambda a, o=None: to_dev(torch, dev, a, o)
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
    130M layer by default), with a seeded dL/dy and no dL/dh_out: the training
    forward (which leaves its states for the backward) and the backward that
    takes them; also the backward that recomputes them."""
    wl = inputs.WORKLOADS[k]
    d = inputs.workload_inputs(k)
    T = d["x"].shape[0]
    nseq = len(d["cu_seqlens"]) - 1
    op = torch.bfloat16
    t = lambda a, dt=None: to_dev(torch, dev, a, dt)
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
    algorithmic bytes and flops."""
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


def copy_calibration(mib):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 10}))


# --------------------------------------------------------- profile summaries
KERNEL_NAMES = {  # kernel symbol fragment -> bench kernel name (first match wins)
    "k_step_multi": "decode_multi_step", "k_conv1d_step": "conv1d_step",
    "k_gated_rmsnorm": "gated_rmsnorm", "k_s6_summary": "s6_summary", "k_s6_pass": "s6_pass",
    "k_s6_replay": "s6_replay", "k_bwd_scan": "bwd_scan", "k_state_pass_bwd": "state_pass_bwd",
    "k_bwd_ddt": "bwd_ddt", "k_bwd_sums": "bwd_sums", "k_gdn_prep": "gdn_chunk_prep",
    "k_gdn_walk": "gdn_chunk_walk", "k_gdn": "gated_delta_rule",
    "k_chunk_state": "chunk_state", "k_state_pass": "state_pass", "k_chunk_scan": "chunk_scan",
    "k_chunk_map": "chunk_map", "k_step": "decode_step", "k_state_walk": "state_walk",
    "k_bfrag": "b_frag", "k_walk_fixup": "walk_fixup",
}
BWD_SCAN_MODES = {"0": "bwd_scan_dx", "1": "bwd_scan_db", "2": "bwd_scan_dc"}
# one profiled bench run per section: its workload name and its command's bench arguments
PROFILED = {
    "headline": ("mamba2-2.7b-layer-prefill",
                 "--sections headline --no-cpu-baseline --no-parity --steps 10 --warmup 2 --quiet"),
    "longctx": ("long-context-varlen-prefill",
                "--sections longctx --no-cpu-baseline --no-parity --quiet"),
    "small": ("mamba2-130m-layer-prefill",
              "--sections small --no-cpu-baseline --no-parity --steps 20 --warmup 2 --quiet"),
    "decode": ("codestral-7b-decode-step",
               "--sections decode --no-cpu-baseline --no-parity --decode-steps 32 --quiet"),
}


PIPE_SECTIONS = ("headline", "small")
PIPE_COUNTERS = (
    ("SQ_WAVE_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
     "SQ_ACTIVE_INST_VALU", "SQ_VMEM_TA_ADDR_FIFO_FULL", "SQ_VALU_MFMA_BUSY_CYCLES"),
    ("TA_BUSY_avr", "TA_ADDR_STALLED_BY_TC_CYCLES_sum", "TCP_PENDING_STALL_CYCLES_sum",
     "TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum", "GRBM_GUI_ACTIVE"),
    ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR",
     "SQ_WAVES", "TCC_HIT_sum", "TCC_MISS_sum"),
)


def _kernel_key(name):
    for frag, k in KERNEL_NAMES.items():
        if frag in name:
            if k == "bwd_scan":  # template mode: k_bwd_scan<T, MODE, ...>
                mode = name.split(frag, 1)[1].split(",")[1].strip() if "<" in name else ""
                k = BWD_SCAN_MODES.get(mode, k)
            if k == "chunk_state" and "true>" in name:
                k = "chunk_state_bwd"
            return k
    return None


def _template_args(name):
    """The integer template arguments of a kernel name, mangled (Li256E) or
    demangled (<64, 128, 256>), as a short suffix such as <64,128,256>."""
    import re
    vals = re.findall(r"Li(\d+)E", name)
    if not vals and "<" in name:
        vals = re.findall(r"\b(\d+)\b", name.split("<", 1)[1].split(">", 1)[0])
    return "<" + ",".join(vals) + ">" if vals else ""


def profile_commands():
    cmds = {}
    for sec, (_, a) in PROFILED.items():
        base = f"-- python bench.py {a}"
        # counters per dispatch do not depend on the clocks: no preheat (its
        # thousands of dispatches would only swell the output)
        pbase = base + " --preheat 0"
        cmds[f"{sec}_trace"] = ("rocprofv3 --kernel-trace --stats --output-format csv "
                                f"-d DIR/{sec}_trace -o run {base}")
        cmds[f"{sec}_fetch"] = f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/{sec}_fetch -o run {pbase}"
        cmds[f"{sec}_write"] = f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/{sec}_write -o run {pbase}"
        cmds[f"{sec}_mfma"] = ("rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 --output-format csv "
                               f"-d DIR/{sec}_mfma -o run {pbase}")
    # where the headline's kernels wait: SQ issue and wait states, the vector
    # memory path (TA address FIFO, L1 pending on L2, L2 read latency), L2 hits
    for sec in PIPE_SECTIONS:
        hb = f"-- python bench.py {PROFILED[sec][1]} --preheat 0"
        for i, cs in enumerate(PIPE_COUNTERS):
            cmds[f"{sec}_pipe{i + 1}"] = (f"rocprofv3 --pmc {' '.join(cs)} --output-format csv "
                                          f"-d DIR/{sec}_pipe{i + 1} -o run {hb}")
    cmds["train_trace"] = ("rocprofv3 --kernel-trace --stats --output-format csv -d DIR/train_trace "
                           "-o run -- python bench.py --train-only --steps 50 --warmup 5 --quiet")
    cmds["cfetch"] = ("rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/cfetch -o run -- "
                      "python bench.py --copy-calibration 1024")
    cmds["cwrite"] = ("rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/cwrite -o run -- "
                      "python bench.py --copy-calibration 1024")
    return cmds


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize(directory):
    """rocprofv3 CSVs under DIR (one sub-directory per command of
    profile_commands(), named by its key) -> profiles/*.txt and
    profiles/traffic.json.  Sections without output are skipped."""
    import glob
    cmds = profile_commands()

    def pmc(sub, counter):
        acc = {}
        for p in glob.glob(os.path.join(directory, sub, "**", "*counter_collection.csv"),
                           recursive=True):
            for r in _read_csv(p):
                if r["Counter_Name"] != counter:
                    continue
                acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return acc

    def copy_factor(sub, counter, nbytes):
        vals = [v for k, vs in pmc(sub, counter).items() for v in vs
                if "copy" in k.lower() or "elementwise" in k.lower()]
        big = [v for v in vals if v * 1024 > nbytes / 4]
        if not big:
            return None
        return nbytes / (float(np.median(big)) * 1024)   # true bytes per counted byte

    f_fac = copy_factor("cfetch", "FETCH_SIZE", 1024 << 20)
    w_fac = copy_factor("cwrite", "WRITE_SIZE", 1024 << 20)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    # the kernel sources the profiled runs were built from, as each run printed
    # them (bench.py prints the hash on every run); all runs must agree
    import re
    seen = set()
    for log_path in glob.glob(os.path.join(directory, "*.log")):
        with open(log_path, errors="replace") as fh:
            seen.update(re.findall(r"bench: kernel sources hash ([0-9a-f]{16})", fh.read()))
    if len(seen) > 1:
        raise SystemExit(f"profiled runs disagree on the kernel sources: {sorted(seen)}")
    if not seen:
        raise SystemExit(f"no 'bench: kernel sources hash' line in {directory}/*.log: the "
                         "profiled runs' output must be kept beside their results")
    traffic = {"source_hash": seen.pop(), "fetch_factor": f_fac, "write_factor": w_fac}
    try:  # keep the figures of sections not profiled this time, if taken on the same sources
        with open(TRAFFIC_FILE) as f:
            old = json.load(f)
        if old.get("source_hash") == traffic["source_hash"]:
            traffic.update({k: v for k, v in old.items() if isinstance(v, dict)})
    except (OSError, ValueError):
        pass
    stamp = f"kernel sources hash {traffic['source_hash']}\n"
    for sec, (wl, _) in PROFILED.items():
        lines = []
        for kind, counter, fac in (("fetch", "FETCH_SIZE", f_fac), ("write", "WRITE_SIZE", w_fac)):
            for kname, vs in sorted(pmc(f"{sec}_{kind}", counter).items()):
                k = _kernel_key(kname)
                if k is None or fac is None:
                    continue
                b = float(np.mean(vs)) * 1024 * fac
                traffic.setdefault(wl, {}).setdefault(k, {})[counter.lower()] = round(b)
                lab = k + _template_args(kname)
                lines.append(f"{lab:30s} {counter:10s} {np.mean(vs):14.1f} KiB/dispatch x "
                             f"{fac:.4f} = {b / 1e6:10.3f} MB ({len(vs)} dispatches)")
        for k, v in traffic.get(wl, {}).items():
            if "fetch_size" in v and "write_size" in v:
                v["bytes"] = v["fetch_size"] + v["write_size"]
        if lines:
            with open(os.path.join(ROOT, "profiles", f"hbm_traffic_{sec}_{wl}.txt"), "w") as f:
                f.write(f"HBM traffic per dispatch, workload {wl}: rocprofv3 FETCH_SIZE and\n"
                        "WRITE_SIZE, each scaled by what the same counter reads over a plain\n"
                        f"1 GiB device copy (true bytes / counted bytes): fetch {f_fac}, "
                        f"write {w_fac}\n{stamp}commands (cwd = repository root, DIR = output "
                        f"directory):\n  {cmds[sec + '_fetch']}\n  {cmds[sec + '_write']}\n"
                        f"  {cmds['cfetch']}\n  {cmds['cwrite']}\n\n" + "\n".join(lines) + "\n")
        mf_util, mf_flops = pmc(f"{sec}_mfma", "MfmaUtil"), pmc(f"{sec}_mfma", "MfmaFlopsBF16")
        if mf_util:
            ml = []
            for kname, vs in sorted(mf_util.items()):
                k = _kernel_key(kname)
                if k is None:
                    continue
                issued = float(np.mean(mf_flops.get(kname, [0.0])))
                ml.append(f"{k + _template_args(kname):30s} MfmaUtil {np.mean(vs):6.2f} %   MfmaFlopsBF16 "
                          f"{issued / 1e9:10.3f} GFLOP/dispatch   ({len(vs)} dispatches)")
            with open(os.path.join(ROOT, "profiles", f"mfma_util_{sec}_{wl}.txt"), "w") as f:
                f.write(f"MFMA utilisation per dispatch, workload {wl}: rocprofv3 derived\n"
                        "counters MfmaUtil = sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max(GRBM_GUI_ACTIVE)\n"
                        "x SIMDs) x 100 and MfmaFlopsBF16 = bf16 MFMA flops issued (padding and\n"
                        f"masked blocks included).\n{stamp}command (cwd = repository root):\n"
                        f"  {cmds[sec + '_mfma']}\n\n" + "\n".join(ml) + "\n")
        _trace_summary(glob.glob(os.path.join(directory, f"{sec}_trace", "**", "*kernel_stats.csv"),
                                 recursive=True),
                       os.path.join(ROOT, "profiles", f"kernel_trace_{sec}_{wl}.txt"),
                       f"rocprofv3 kernel trace, workload {wl}\n{stamp}command (cwd = repository "
                       f"root):\n  {cmds[sec + '_trace']}\n")
    for sec in PIPE_SECTIONS:
        _pipeline_summary(directory, cmds, pmc, stamp, sec)
    _trace_summary(glob.glob(os.path.join(directory, "train_trace", "**", "*kernel_stats.csv"),
                             recursive=True),
                   os.path.join(ROOT, "profiles", "kernel_trace_train_mamba2-130m-layer.txt"),
                   "rocprofv3 kernel trace of forward + backward of the Mamba-2 130M layer scan\n"
                   "(4096 tokens, 24 heads, P 64, N 128, chunk 256, bf16, h0 = 0, dL/dh_out = 0)\n"
                   f"{stamp}command (cwd = repository root):\n  {cmds['train_trace']}\n")
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(traffic, f, indent=1)
    print(json.dumps(traffic, indent=1))


def _pipeline_summary(directory, cmds, pmc, stamp, sec):
    """profiles/memory_pipeline_<sec>_<workload>.txt from the <sec>_pipe*
    counter runs: per kernel, fractions of wave time and of the kernel's
    duration per XCD, and the L1's average wait for L2 reads."""
    wl = PROFILED[sec][0]
    vals = {}
    for i, cs in enumerate(PIPE_COUNTERS):
        for c in cs:
            for kname, vs in pmc(f"{sec}_pipe{i + 1}", c).items():
                k = _kernel_key(kname)
                if k is not None:
                    vals.setdefault(k, {})[c] = float(np.mean(vs))
    if not vals:
        return
    lines = []
    for k, v in sorted(vals.items()):
        wc = v.get("SQ_WAVE_CYCLES") or 0.0
        xcd_cycles = (v.get("GRBM_GUI_ACTIVE") or 0.0) / 8.0  # summed over the 8 XCDs
        f = lambda c: v.get(c, 0.0) / wc if wc else float("nan")
        per_cu = lambda c: v.get(c, 0.0) / 256.0 / xcd_cycles if xcd_cycles else float("nan")
        lat = (v.get("TCP_TCC_READ_REQ_LATENCY_sum", 0.0) / v["TCP_TCC_READ_REQ_sum"]
               if v.get("TCP_TCC_READ_REQ_sum") else float("nan"))
        hit = v.get("TCC_HIT_sum", 0.0) / max(1.0, v.get("TCC_HIT_sum", 0.0) + v.get("TCC_MISS_sum", 0.0))
        waves = max(1.0, v.get("SQ_WAVES", 1.0))
        lines.append(
            f"{k:14s} wave time: waiting {f('SQ_WAIT_ANY'):.2f}  issue-blocked {f('SQ_WAIT_INST_ANY'):.2f}"
            f"  issuing {f('SQ_ACTIVE_INST_ANY'):.2f} (VALU {f('SQ_ACTIVE_INST_VALU'):.2f}, MFMA busy "
            f"{f('SQ_VALU_MFMA_BUSY_CYCLES'):.2f})\n"
            f"{'':14s} per CU, of the kernel's time: L1 waiting on L2 data "
            f"{per_cu('TCP_PENDING_STALL_CYCLES_sum'):.2f}, TA stalled by L1 "
            f"{per_cu('TA_ADDR_STALLED_BY_TC_CYCLES_sum'):.2f}, TA busy "
            f"{v.get('TA_BUSY_avr', 0.0) / xcd_cycles if xcd_cycles else float('nan'):.2f}\n"
            f"{'':14s} L2 read latency seen by L1 {lat:.0f} cycles, L2 hit rate {hit:.2f}; per wave: "
            f"VALU {v.get('SQ_INSTS_VALU', 0) / waves:.0f}, MFMA {v.get('SQ_INSTS_MFMA', 0) / waves:.0f}, "
            f"LDS {v.get('SQ_INSTS_LDS', 0) / waves:.0f}, loads {v.get('SQ_INSTS_VMEM_RD', 0) / waves:.0f}, "
            f"stores {v.get('SQ_INSTS_VMEM_WR', 0) / waves:.0f} instructions")
    with open(os.path.join(ROOT, "profiles", f"memory_pipeline_{sec}_{wl}.txt"), "w") as fh:
        fh.write(f"Where the kernels of workload {wl} wait: rocprofv3 counters per dispatch\n"
                 "(SQ_* summed over the waves, TA/TCP summed over the 256 CUs, GRBM_GUI_ACTIVE over\n"
                 f"the 8 XCDs).\n{stamp}commands (cwd = repository root, DIR = output directory):\n"
                 + "".join(f"  {cmds[f'{sec}_pipe{i + 1}']}\n" for i in range(len(PIPE_COUNTERS)))
                 + "\n" + "\n".join(lines) + "\n")


def _trace_summary(stats, out, head):
    if not stats:
        return
    tl = []
    for r in _read_csv(stats[0]):
        tl.append(f"{r['Name'][:96]:96s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f}"
                  f" {float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f}"
                  f" {float(r['Percentage']):6.2f}")
    with open(out, "w") as f:
        f.write(head + f"\n{'kernel':96s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"
                f" {'%':>6s}\n" + "\n".join(tl) + "\n")


# ---------------------------------------------------------------------- main
def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize)
        return
    print(f"bench: kernel sources hash {source_hash()}", file=sys.stderr, flush=True)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): this library runs on "
              "one GPU and has no multi-GPU path; run it with --gpus 1", file=sys.stderr)
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
    sec = set(args.sections)
    # the headline's inputs are built first and its timing runs last, right
    # after the other sections' GPU work (it still gets its own warm-up steps)
    go_headline = headline(args, torch, inputs, ssd, dev) if "headline" in sec else None
    rest = {}
    if "small" in sec:
        rest["prefill_130m_layer"] = small_layer(args, torch, inputs, ssd, dev)
    if "longctx" in sec:
        rest["prefill_long_context_varlen"] = long_context_bench(args, torch, inputs, ssd, dev)
    if "decode" in sec:
        rest["decode"], rest["decode_multi_step"], rest["decode_layer_step"] = \
            decode_bench(args, torch, inputs, ssd, dev)
    if "s6" in sec:
        rest["selective_scan_w1"] = selective_scan_bench(torch, inputs, ssd, dev)
    if "gdn" in sec:
        rest["gated_delta_rule"] = gdn_bench(torch, inputs, ssd, dev)
    if "train" in sec:
        rest["training_step_130m"] = training_step_bench(args, torch, inputs, ssd, dev)
        rest["training_step_2p7b"] = training_step_bench(args, torch, inputs, ssd, dev, k=2)
    out = {"metric": "SSD prefill tokens/s + MFMA util; decode state-update GB/s vs HBM peak"}
    hl = go_headline() if go_headline is not None else None
    if hl is not None:
        dom = hl["dominant"]
        out.update({
            "value": round(hl["value"], 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(hl["ms_step"], 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic", "config": hl["config"],
            "roofline": {k: dom[k] for k in ("bound", "achieved", "peak", "unit", "frac",
                                             "traffic")} | {"kernel": dom["kernel"],
                                                            "avg_us": dom["avg_us"]},
            "ms_per_step_graph": round(hl["ms_step_graph"], 5),
            "preheat": hl["preheat"],
            "prefill": hl["prefill"],
            "prefill_mfma_util": hl["prefill"]["mfma_frac"],
            "kernels": hl["kernels"],
            "parity": hl["parity"],
        })
    out.update(rest)
    out["cpu_baseline"] = hl["cpu"] if hl is not None else None
    out["provenance"] = provenance(torch)
    print(json.dumps(out), flush=True)
    if hl is not None and hl["parity"] is not None and not hl["parity"]["ok"]:
        print("parity check of the timed outputs FAILED", file=sys.stderr)
        sys.exit(1)


if __name__ == "__main__":
    main()
