"""GPU chunked prefill (ssd_scan_prefill through the C ABI) against the fp64
oracle, plus the invariants that hold on the GPU itself.

Every workload test compares every element of y and h_out with one full
oracle run (max-abs 2e-2 in bfloat16 mode, 1e-4 in float32 mode), and in
bfloat16 mode also bounds the error relative to the size of the state-space
part of the output, max|dy| / max|y_ref - D x| <= 1e-2 (the skip term D x
dominates |y|, so the absolute bound alone tests the state path loosely)."""
import numpy as np
import pytest

import oracle
from gpu_util import SSM_REL_TOL, TOL, dev_inputs, log, maxabs, ssm_scale
from state_space_model_amd import inputs

pytestmark = pytest.mark.gpu

SCANS = ("auto", "rows", "heads")
STATES = ("chunks", "walk")   # how the chunk states are formed and carried


def _gpu(d, dtype, chunk, with_h0=True, scan="auto", state="auto", **kw):
    import torch
    from state_space_model_amd import ssd
    t = dev_inputs(d, dtype)
    y, ho = ssd.prefill(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"],
                        t["h0"] if with_h0 else None, chunk=chunk,
                        cu_seqlens=t["cu_seqlens"], scan=scan, state=state, **kw)
    torch.cuda.synchronize()
    out = y.cpu().numpy(), ho.cpu().numpy()
    del y, ho, t
    return out


def _ref(d, with_h0=True):
    h0 = d["h0"].astype(np.float64) if (with_h0 and d.get("h0") is not None) else None
    return oracle.prefill(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], h0, d["cu_seqlens"])


def _check(what, y, ho, ry, rh, tol, ssm=None):
    """Every element of y and h_out against the oracle; with `ssm` (the size
    of the state-space part of y) also the relative bound."""
    ey, eh = maxabs(y, ry), maxabs(ho, rh)
    rel = "" if ssm is None else f" max|dy|/max|y_ssm|={ey / max(ssm, 1e-30):.3g}"
    log(f"  {what}: max|dy|={ey:.3g} max|dh|={eh:.3g}{rel}")
    assert ey <= tol and eh <= tol, (what, ey, eh)
    if ssm is not None:
        assert ey <= SSM_REL_TOL * ssm, (what, ey, ssm)
    return ey, eh


SMALL = [  # (lengths, H, P, N, G, chunk, h0)
    ([200], 4, 16, 16, 1, 64, False),
    ([300], 2, 32, 32, 1, 32, True),
    ([257, 3, 130], 4, 64, 128, 2, 64, True),
    ([1000], 3, 64, 64, 3, 128, True),
    ([520, 0, 77], 4, 128, 16, 4, 256, True),
    ([1100, 513], 2, 64, 128, 1, 512, True),
    ([96], 8, 16, 128, 8, 32, False),
    ([130, 45], 4, 64, 128, 2, 32, True),   # block-swizzled tiles at chunk 32 (two waves)
    ([300, 129, 77], 4, 64, 128, 2, 128, True),  # C.B^T per (chunk, group) at chunk 128
    ([700, 1, 300], 6, 64, 128, 3, 256, True),   # ... and at chunk 256, three groups
    ([900, 0, 350, 1], 4, 64, 128, 1, 64, False),  # no h0: the walk's cut chains from zero
]


MODES = [("f32", "auto", "auto"), ("bf16", "rows", "chunks"), ("bf16", "heads", "chunks"),
         ("bf16", "rows", "walk"), ("bf16", "heads", "walk")]


@pytest.mark.parametrize("dtype,scan,state", MODES)
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_prefill_small(dtype, scan, state, case):
    """Every small shape in float32, and in bfloat16 through both chunk-scan
    kernels (row-split, and heads streamed where a shape has that kernel) and
    both ways of forming the states (chunk states, and the walk where a shape
    has it)."""
    lengths, H, P, N, G, chunk, h0 = SMALL[case]
    log(f"prefill small dtype={dtype} scan={scan} state={state} lengths={lengths} H={H} P={P}"
        f" N={N} G={G} Q={chunk}")
    d = inputs.prefill_inputs(H, P, N, G, lengths, 200 + case, dtype=dtype, h0=h0)
    y, ho = _gpu(d, dtype, chunk, scan=scan, state=state)
    ry, rh = _ref(d)
    _check(f"{dtype} {scan} {state}", y, ho, ry, rh, TOL[dtype])


# (lengths, dense, H, G, chunk): dense batches walk in segments, packed ones by
# lists (runs of 8 or more chunk positions, cutting chains where they end)
WALK_SEGMENT_CASES = [
    ([3000, 0, 40, 1500, 64], False, 8, 2, 64),  # empty, one-chunk, exactly one-chunk sequences
    ([571, 571], True, 8, 1, 64),                # 9 chunks a sequence: segments of 4 and 5
    ([2100, 700, 1], False, 6, 3, 128),          # one token alone in its segment pair
    # chunk 256, the layer shapes' chunk
    ([4000, 0, 300, 3500], False, 8, 1, 256),    # empty sequence, one-chunk segments
    ([2400, 2400], True, 8, 2, 256),             # 10 chunks a sequence, two groups
    # more chains than the chip holds at once with two segments each: the
    # first heads in two segments, the rest in shorter ones
    ([2048, 2048], True, 160, 1, 256),
    ([3000, 1, 2600], False, 100, 2, 256),
    # more chunk positions than 8 per resident workgroup: longer runs, a
    # one-chunk chain between two cut ones
    ([2000, 1500, 37], False, 80, 1, 64),
]


@pytest.mark.parametrize("scan", ["rows", "heads"])
@pytest.mark.parametrize("case", range(len(WALK_SEGMENT_CASES)))
def test_prefill_walk_segments(case, scan):
    """The state walk cuts chains into pieces walked at once (each after a
    chain's first from a zero state) and corrects the later pieces' entering
    states and the final state afterwards -- dense batches in segments per
    head, packed batches by runs of chunk positions: packed batches with
    empty, one-chunk and one-token sequences, and dense batches with odd and
    even chunk counts, through both chunk-scan kernels, every element against
    the oracle, as are the chunk-parallel states on the same batch and each
    packed sequence run alone (which may walk unsegmented); the stages run
    one by one equal one call, bitwise."""
    import torch
    from state_space_model_amd import ssd
    lengths, dense, H, G, chunk = WALK_SEGMENT_CASES[case]
    log(f"prefill walk segments: lengths={lengths} dense={dense} H={H} G={G} Q={chunk}"
        f" scan={scan}")
    d = inputs.prefill_inputs(H, 64, 128, G, lengths, 5100 + case, dtype="bf16", h0=True)
    ry, rh = _ref(d)
    t = dev_inputs(d, "bf16")
    kw = dict(nseq=len(lengths)) if dense else dict(cu_seqlens=t["cu_seqlens"])
    kw.update(chunk=chunk, scan=scan)
    args = (t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"])
    y, ho = ssd.prefill(*args, state="walk", **kw)
    yc, hc = ssd.prefill(*args, state="chunks", **kw)
    ws = ssd.alloc_workspace(sum(lengths), len(lengths), H, 64, 128, G, chunk, torch.bfloat16,
                             "cuda")
    y2, h2 = torch.empty_like(y), torch.empty_like(ho)
    for st in (1, 2, 4, 8):
        ssd.prefill(*args, y=y2, h_out=h2, workspace=ws, stages=st, state="walk", **kw)
    torch.cuda.synchronize()
    _check("walk, cut chains", y.cpu().numpy(), ho.cpu().numpy(), ry, rh, TOL["bf16"])
    _check("chunk states", yc.cpu().numpy(), hc.cpu().numpy(), ry, rh, TOL["bf16"])
    assert torch.equal(y, y2) and torch.equal(ho, h2)
    if not dense:  # each sequence alone (one sequence: cut by its own runs)
        cu = d["cu_seqlens"]
        for k in range(len(lengths)):
            a, b = int(cu[k]), int(cu[k + 1])
            one = torch.tensor([0, b - a], dtype=torch.int32, device="cuda")
            ys, hs = ssd.prefill(t["x"][a:b].contiguous(), t["dt"][a:b].contiguous(), t["A"],
                                 t["B"][a:b].contiguous(), t["C"][a:b].contiguous(), t["D"],
                                 t["h0"][k:k + 1].contiguous(), chunk=chunk, state="walk",
                                 scan=scan, cu_seqlens=one)
            torch.cuda.synchronize()
            err = (maxabs(ys.cpu().numpy(), ry[a:b]), maxabs(hs.cpu().numpy(), rh[k:k + 1]))
            assert max(err) <= TOL["bf16"], (k, err)


def test_prefill_heads_streamed_several_heads_per_workgroup():
    """80 heads in 2 groups at chunk 256 over a packed pair of ragged
    sequences (17 chunks x 80 heads): on the heads-streamed scan the head-count
    rule gives each workgroup 8 heads of a group, so the next-head loads, the
    buffer swap and the shared C.B^T all run; on the row-split scan (1360
    units, C.B^T precomputed per chunk and group) every element is checked
    against the oracle too."""
    lengths, H, P, N, G, chunk = [2500, 1596], 80, 64, 128, 2, 256
    log(f"prefill heads streamed, several heads per workgroup: lengths={lengths} H={H} G={G}")
    d = inputs.prefill_inputs(H, P, N, G, lengths, 4242, dtype="bf16", h0=True)
    ry, rh = _ref(d)
    ssm = ssm_scale(ry, d["x"], d["D"])
    for state in STATES:
        y, ho = _gpu(d, "bf16", chunk, scan="heads", state=state)
        _check(f"heads {state}", y, ho, ry, rh, TOL["bf16"], ssm)
        y2, ho2 = _gpu(d, "bf16", chunk, scan="rows", state=state)
        _check(f"rows {state}", y2, ho2, ry, rh, TOL["bf16"], ssm)
        assert maxabs(ho, ho2) == 0.0  # the state path is the same kernels in both


def test_prefill_tiny_workload_f32():
    w = inputs.WORKLOADS[0]
    log("prefill workload 0 (tiny, float32)")
    d = inputs.workload_inputs(0)
    y, ho = _gpu(d, "f32", w.chunk)
    ry, rh = _ref(d)
    _check("f32", y, ho, ry, rh, TOL["f32"])


def _workload_all_elements(k, scans, d_zero=False, states=STATES):
    """Workload k: one full oracle run, every element of y and h_out compared
    for each chunk-scan kernel and each way of forming the states; with d_zero
    the skip term is removed (D = 0), so y is the state-space part alone."""
    w = inputs.WORKLOADS[k]
    d = inputs.workload_inputs(k)
    ry, rh = _ref(d)
    if d_zero:
        # the oracle's y is sum_n C h + D x: with D = 0 it is that sum, which
        # is ry - D x up to one float64 rounding
        ry = ry - d["D"][None, :, None].astype(np.float64) * d["x"]
        d = dict(d, D=np.zeros_like(d["D"]))
    ssm = ssm_scale(ry, d["x"], d["D"])
    log(f"  oracle done: max|y_ssm|={ssm:.3g}")
    for state in states:
        for scan in scans:
            y, ho = _gpu(d, "bf16", w.chunk, scan=scan, state=state)
            _check(f"scan={scan} state={state}{' D=0' if d_zero else ''}", y, ho, ry, rh,
                   TOL["bf16"], ssm)
            del y, ho


def test_prefill_130m_layer_workload():
    log("prefill workload 1 (Mamba-2 130M layer, bf16), every element, every scan kernel")
    _workload_all_elements(1, SCANS)


def test_prefill_130m_layer_workload_no_skip():
    log("prefill workload 1 with D = 0 (y is the state-space part alone)")
    _workload_all_elements(1, SCANS, d_zero=True)


def test_prefill_2p7b_layer_workload():
    """4 x 8192 tokens, 80 heads, h0 given: every head of every sequence
    against one full oracle run, through both chunk-scan kernels."""
    log("prefill workload 2 (Mamba-2 2.7B layer, bf16), every element, both scan kernels")
    _workload_all_elements(2, ("auto", "rows"))


def test_prefill_2p7b_layer_workload_no_skip():
    log("prefill workload 2 with D = 0 (y is the state-space part alone)")
    _workload_all_elements(2, ("auto",), d_zero=True, states=("auto",))


def test_prefill_long_context_varlen_chunk_sweep():
    """8 packed sequences of 1K-32K tokens with their own h0: every chunk size
    through both chunk-scan kernels, every element against one oracle run."""
    w = inputs.WORKLOADS[4]
    d = inputs.workload_inputs(4)
    lens = np.diff(d["cu_seqlens"])
    log(f"prefill workload 4 (varlen, lengths {lens.tolist()}), chunks {w.chunks}")
    ry, rh = _ref(d)
    ssm = ssm_scale(ry, d["x"], d["D"])
    log(f"  oracle done: max|y_ssm|={ssm:.3g}")
    for state in STATES:
        for scan in ("auto", "rows"):
            for q in w.chunks:
                y, ho = _gpu(d, "bf16", q, scan=scan, state=state)
                _check(f"scan={scan} state={state} Q={q}", y, ho, ry, rh, TOL["bf16"], ssm)
                del y, ho


# ---- the method's closed forms and degenerate cases, through the kernels, at
# the Mamba-2 130M layer shape (4096 tokens, 24 heads, P 64, N 128, chunk 256)

def _layer_inputs(seed, dtype, h0=True):
    return inputs.prefill_inputs(24, 64, 128, 1, [4096], seed, dtype=dtype, h0=h0)


@pytest.mark.parametrize("dtype,scan,state", MODES)
def test_prefill_no_decay_is_a_prefix_sum(dtype, scan, state):
    """A = 0: no decay, the state is h0 plus the running sum of dt x (x) B.
    float32 within 1e-4 of the output's scale, bfloat16 within 2e-2."""
    d = _layer_inputs(61, dtype)
    d["A"] = np.zeros_like(d["A"])
    log(f"prefill A=0 dtype={dtype} scan={scan} state={state}")
    ry, rh = _ref(d)
    scale = max(1.0, float(np.max(np.abs(ry))), float(np.max(np.abs(rh))))
    y, ho = _gpu(d, dtype, 256, scan=scan, state=state)
    _check(f"A=0 {dtype} {scan} {state} (scale {scale:.3g})", y, ho, ry, rh, TOL[dtype] * scale)


@pytest.mark.parametrize("dtype,scan,state", MODES)
def test_prefill_zero_step_keeps_the_state(dtype, scan, state):
    """dt = 0: nothing enters and nothing decays, so h_out equals h0 bit for
    bit and y = C h0 + D x."""
    d = _layer_inputs(62, dtype)
    d["dt"] = np.zeros_like(d["dt"])
    log(f"prefill dt=0 dtype={dtype} scan={scan} state={state}")
    ry, rh = _ref(d)
    y, ho = _gpu(d, dtype, 256, scan=scan, state=state)
    assert np.array_equal(ho, d["h0"]), "h_out differs from h0 with dt = 0"
    ssm = ssm_scale(ry, d["x"], d["D"]) if dtype == "bf16" else None
    _check(f"dt=0 {dtype} {scan} {state}", y, ho, ry, rh, TOL[dtype], ssm)


@pytest.mark.parametrize("dtype,scan,state", MODES)
def test_prefill_strong_decay(dtype, scan, state):
    """A = -16 with dt in [0.5, 1]: every step decays the state by 1e-7 to
    3e-4 and a chunk's decay underflows to zero (the fully decayed regime)."""
    d = _layer_inputs(63, dtype)
    rng = np.random.Generator(np.random.PCG64(64))
    d["A"] = np.full_like(d["A"], -16.0)
    d["dt"] = rng.uniform(0.5, 1.0, size=d["dt"].shape).astype(np.float32)
    log(f"prefill strong decay dtype={dtype} scan={scan} state={state}")
    ry, rh = _ref(d)
    y, ho = _gpu(d, dtype, 256, scan=scan, state=state)
    ssm = ssm_scale(ry, d["x"], d["D"]) if dtype == "bf16" else None
    _check(f"strong decay {dtype} {scan} {state}", y, ho, ry, rh, TOL[dtype], ssm)


def test_stages_separately_equal_one_call():
    import torch
    from state_space_model_amd import ssd
    d = inputs.prefill_inputs(4, 64, 128, 1, [700, 300], 5, dtype="bf16", h0=True)
    t = dev_inputs(d, "bf16")
    args = (t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"])
    for scan in SCANS:
        for state in STATES:
            kw = dict(chunk=128, cu_seqlens=t["cu_seqlens"], scan=scan, state=state)
            y1, h1 = ssd.prefill(*args, **kw)
            ws = ssd.alloc_workspace(1000, 2, 4, 64, 128, 1, 128, torch.bfloat16, "cuda")
            y2 = torch.empty_like(y1)
            h2 = torch.empty_like(h1)
            for st in (1, 2, 4, 8):
                ssd.prefill(*args, y=y2, h_out=h2, workspace=ws, stages=st, **kw)
            torch.cuda.synchronize()
            assert torch.equal(y1, y2) and torch.equal(h1, h2), (scan, state)
            # h_out may be the h0 buffer itself, also with the stages run one by one
            hbuf = t["h0"].clone()
            for st in (1, 2, 4, 8):
                ssd.prefill(*args[:6], hbuf, y=y2, h_out=hbuf, workspace=ws, stages=st, **kw)
            torch.cuda.synchronize()
            assert torch.equal(y1, y2) and torch.equal(h1, hbuf), (scan, state)


@pytest.mark.parametrize("state", STATES)
@pytest.mark.parametrize("scan", ["rows", "heads"])
def test_deterministic_and_varlen_equals_solo(scan, state):
    """Run-to-run bitwise determinism; a packed batch equals each sequence run
    alone, bitwise; h_out may be the h0 buffer itself.  (The walk by lists
    cuts a packed batch's chains where its runs of 8 chunk positions end;
    here each run holds whole chains -- 4 heads x 2, 1 + 1, and 2 x 4 chunks
    -- so nothing is rounded twice and the equality is exact.)"""
    import torch
    from state_space_model_amd import ssd
    lengths = [333, 64, 1, 900]
    d = inputs.prefill_inputs(4, 64, 128, 2, lengths, 9, dtype="bf16", h0=True)
    t = dev_inputs(d, "bf16")
    run = lambda: ssd.prefill(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"],
                              chunk=256, cu_seqlens=t["cu_seqlens"], scan=scan, state=state)
    y1, h1 = run()
    y2, h2 = run()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
    cu = d["cu_seqlens"]
    for s in range(len(lengths)):
        sl = slice(int(cu[s]), int(cu[s + 1]))
        ys, hs = ssd.prefill(t["x"][sl], t["dt"][sl], t["A"], t["B"][sl], t["C"][sl], t["D"],
                             t["h0"][s:s + 1].contiguous(), chunk=256, scan=scan, state=state)
        assert torch.equal(ys, y1[sl]) and torch.equal(hs[0], h1[s])
    hbuf = t["h0"].clone()
    y3, _ = ssd.prefill(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], hbuf, chunk=256,
                        cu_seqlens=t["cu_seqlens"], h_out=hbuf, scan=scan, state=state)
    torch.cuda.synchronize()
    assert torch.equal(y3, y1) and torch.equal(hbuf, h1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_hands_state_on(dtype):
    import torch
    from state_space_model_amd import ssd
    L, k = 1000, 377
    d = inputs.prefill_inputs(2, 64, 64, 1, [L], 13, dtype=dtype, h0=True)
    t = dev_inputs(d, dtype)
    f = lambda sl, h0: ssd.prefill(t["x"][sl], t["dt"][sl], t["A"], t["B"][sl], t["C"][sl], t["D"],
                                   h0, chunk=128)
    y, h = f(slice(0, L), t["h0"])
    y1, h1 = f(slice(0, k), t["h0"])
    y2, h2 = f(slice(k, L), h1)
    torch.cuda.synchronize()
    assert maxabs(torch.cat([y1, y2]).cpu(), y.cpu()) <= TOL[dtype]
    assert maxabs(h2.cpu(), h.cpu()) <= TOL[dtype]


def test_prefill_equals_steps():
    import torch
    from state_space_model_amd import ssd
    L = 150
    d = inputs.prefill_inputs(4, 32, 64, 2, [L], 17, dtype="f32", h0=True)
    t = dev_inputs(d, "f32")
    y, h = ssd.prefill(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], chunk=64)
    hs = t["h0"].clone()
    ys = [ssd.step(t["x"][i:i + 1], t["dt"][i:i + 1], t["A"], t["B"][i:i + 1], t["C"][i:i + 1],
                   t["D"], hs) for i in range(L)]
    torch.cuda.synchronize()
    assert maxabs(torch.cat(ys).cpu(), y.cpu()) <= TOL["f32"]
    assert maxabs(hs.cpu(), h.cpu()) <= TOL["f32"]


def test_empty_and_aliasing():
    import torch
    from state_space_model_amd import ssd
    d = inputs.prefill_inputs(4, 16, 32, 1, [0, 0], 19, dtype="f32", h0=True)
    t = dev_inputs(d, "f32")
    y, ho = ssd.prefill(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], chunk=64,
                        cu_seqlens=t["cu_seqlens"])
    torch.cuda.synchronize()
    assert y.numel() == 0 and torch.equal(ho, t["h0"])
    # h_out may be the same buffer as h0
    d = inputs.prefill_inputs(4, 16, 32, 1, [100, 50], 21, dtype="f32", h0=True)
    t = dev_inputs(d, "f32")
    y1, h1 = ssd.prefill(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], chunk=32,
                         cu_seqlens=t["cu_seqlens"])
    hbuf = t["h0"].clone()
    y2, h2 = ssd.prefill(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], hbuf, chunk=32,
                         cu_seqlens=t["cu_seqlens"], h_out=hbuf)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, hbuf)
