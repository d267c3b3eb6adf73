"""GPU chunked prefill (ssd_scan_prefill through the C ABI) against the fp64
oracle, plus the invariants that hold on the GPU itself."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, dev_inputs, log, maxabs, select_heads
from state_space_model_amd import inputs

pytestmark = pytest.mark.gpu


class kernels:
    """Force the chunk-scan kernel for a block (SSD_PREFILL_SCAN=heads|rows);
    "auto" leaves the library's choice."""

    def __init__(self, scan="auto"):
        self.want = {"SSD_PREFILL_SCAN": scan}

    def __enter__(self):
        import os
        self.old = {k: os.environ.get(k) for k in self.want}
        for k, v in self.want.items():
            if v == "auto":
                os.environ.pop(k, None)
            else:
                os.environ[k] = v

    def __exit__(self, *exc):
        import os
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _gpu(d, dtype, chunk, with_h0=True, **kw):
    import torch
    from state_space_model_amd import ssd
    t = dev_inputs(d, dtype)
    y, ho = ssd.prefill(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"],
                        t["h0"] if with_h0 else None, chunk=chunk,
                        cu_seqlens=t["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy(), ho.cpu().numpy()


def _ref(d, with_h0=True):
    h0 = d["h0"].astype(np.float64) if (with_h0 and d.get("h0") is not None) else None
    return oracle.prefill(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], h0, d["cu_seqlens"])


SMALL = [  # (lengths, H, P, N, G, chunk, h0)
    ([200], 4, 16, 16, 1, 64, False),
    ([300], 2, 32, 32, 1, 32, True),
    ([257, 3, 130], 4, 64, 128, 2, 64, True),
    ([1000], 3, 64, 64, 3, 128, True),
    ([520, 0, 77], 4, 128, 16, 4, 256, True),
    ([1100, 513], 2, 64, 128, 1, 512, True),
    ([96], 8, 16, 128, 8, 32, False),
    ([130, 45], 4, 64, 128, 2, 32, True),  # block-swizzled tiles at chunk 32 (two waves)
]


MODES = [("f32", "auto"), ("bf16", "rows"), ("bf16", "heads")]


@pytest.mark.parametrize("dtype,scan", MODES)
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_prefill_small(dtype, scan, case):
    """Every small shape in float32, and in bfloat16 through both chunk-scan
    kernels (row-split, and heads streamed where a shape has that kernel)."""
    lengths, H, P, N, G, chunk, h0 = SMALL[case]
    log(f"prefill small dtype={dtype} scan={scan} lengths={lengths} H={H} P={P} N={N} G={G}"
        f" Q={chunk}")
    d = inputs.prefill_inputs(H, P, N, G, lengths, 200 + case, dtype=dtype, h0=h0)
    with kernels(scan):
        y, ho = _gpu(d, dtype, chunk)
    ry, rh = _ref(d)
    ey, eh = maxabs(y, ry), maxabs(ho, rh)
    log(f"  max|dy|={ey:.3g} max|dh|={eh:.3g}")
    assert ey <= TOL[dtype] and eh <= TOL[dtype]


def test_prefill_heads_streamed_several_heads_per_workgroup():
    """80 heads in 2 groups at chunk 256 over a packed pair of ragged
    sequences (17 chunks x 80 heads): forced onto the heads-streamed scan, the
    head-count rule gives each workgroup 8 heads of a group, so the next-head
    loads, the buffer swap and the shared C.B^T all run; checked against the
    full oracle in bfloat16 and against the row-split scan."""
    lengths, H, P, N, G, chunk = [2500, 1596], 80, 64, 128, 2, 256
    log(f"prefill heads streamed, several heads per workgroup: lengths={lengths} H={H} G={G}")
    d = inputs.prefill_inputs(H, P, N, G, lengths, 4242, dtype="bf16", h0=True)
    with kernels("heads"):
        y, ho = _gpu(d, "bf16", chunk)
    with kernels("rows"):
        y2, ho2 = _gpu(d, "bf16", chunk)
    ry, rh = _ref(d)
    ey, eh = maxabs(y, ry), maxabs(ho, rh)
    log(f"  max|dy|={ey:.3g} max|dh|={eh:.3g} vs rows {maxabs(y, y2):.3g}")
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]
    assert maxabs(ho, ho2) == 0.0  # the state path is the same kernels in both


def test_prefill_tiny_workload_f32():
    w = inputs.WORKLOADS[0]
    log("prefill workload 0 (tiny, float32)")
    d = inputs.workload_inputs(0)
    y, ho = _gpu(d, "f32", w.chunk)
    ry, rh = _ref(d)
    ey, eh = maxabs(y, ry), maxabs(ho, rh)
    log(f"  max|dy|={ey:.3g} max|dh|={eh:.3g}")
    assert ey <= TOL["f32"] and eh <= TOL["f32"]


def test_prefill_130m_layer_workload():
    w = inputs.WORKLOADS[1]
    log("prefill workload 1 (Mamba-2 130M layer, bf16), full oracle, both scan kernels")
    d = inputs.workload_inputs(1)
    ry, rh = _ref(d)
    ssm = np.max(np.abs(ry - d["D"][None, :, None] * d["x"]))
    for scan in ("auto", "heads"):
        with kernels(scan):
            y, ho = _gpu(d, "bf16", w.chunk)
        ey, eh = maxabs(y, ry), maxabs(ho, rh)
        log(f"  scan={scan}: max|dy|={ey:.3g} max|dh|={eh:.3g} (max|y_ssm|={ssm:.3g})")
        assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def test_prefill_2p7b_layer_workload():
    """4 x 8192 tokens, 80 heads: the GPU runs the whole workload; the oracle
    recomputes a sample of heads over every token of every sequence."""
    w = inputs.WORKLOADS[2]
    log("prefill workload 2 (Mamba-2 2.7B layer, bf16), sampled heads, both scan kernels")
    d = inputs.workload_inputs(2)
    heads = [0, 41, 79]
    ds = select_heads(d, heads, w.G)
    ry, rh = _ref(ds)
    for scan in ("auto", "rows"):
        with kernels(scan):
            y, ho = _gpu(d, "bf16", w.chunk)
        ey, eh = maxabs(y[:, heads], ry), maxabs(ho[:, heads], rh)
        log(f"  scan={scan}: max|dy|={ey:.3g} max|dh|={eh:.3g}")
        assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def test_prefill_long_context_varlen_chunk_sweep():
    """8 packed sequences of 1K-32K tokens with their own h0, every chunk size."""
    w = inputs.WORKLOADS[4]
    d = inputs.workload_inputs(4)
    lens = np.diff(d["cu_seqlens"])
    log(f"prefill workload 4 (varlen, lengths {lens.tolist()}), chunks {w.chunks}")
    heads = [3, 66]
    ds = select_heads(d, heads, w.G)
    ry, rh = _ref(ds)
    for scan in ("auto", "rows"):
        for q in w.chunks:
            with kernels(scan):
                y, ho = _gpu(d, "bf16", q)
            ey, eh = maxabs(y[:, heads], ry), maxabs(ho[:, heads], rh)
            log(f"  scan={scan} Q={q}: max|dy|={ey:.3g} max|dh|={eh:.3g}")
            assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def test_stages_separately_equal_one_call():
    import torch
    from state_space_model_amd import ssd
    d = inputs.prefill_inputs(4, 64, 128, 1, [700, 300], 5, dtype="bf16", h0=True)
    t = dev_inputs(d, "bf16")
    args = (t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"])
    y1, h1 = ssd.prefill(*args, chunk=128, cu_seqlens=t["cu_seqlens"])
    ws = ssd.alloc_workspace(1000, 2, 4, 64, 128, 128, torch.bfloat16, "cuda")
    y2 = torch.empty_like(y1)
    h2 = torch.empty_like(h1)
    for st in (1, 2, 4, 8):
        ssd.prefill(*args, chunk=128, cu_seqlens=t["cu_seqlens"], y=y2, h_out=h2, workspace=ws,
                    stages=st)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


@pytest.mark.parametrize("scan", ["rows", "heads"])
def test_deterministic_and_varlen_equals_solo(scan):
    """Run-to-run bitwise determinism; a packed batch equals each sequence run
    alone, bitwise; h_out may be the h0 buffer itself."""
    import torch
    from state_space_model_amd import ssd
    lengths = [333, 64, 1, 900]
    d = inputs.prefill_inputs(4, 64, 128, 2, lengths, 9, dtype="bf16", h0=True)
    t = dev_inputs(d, "bf16")
    with kernels(scan):
        run = lambda: ssd.prefill(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"],
                                  chunk=256, cu_seqlens=t["cu_seqlens"])
        y1, h1 = run()
        y2, h2 = run()
        assert torch.equal(y1, y2) and torch.equal(h1, h2)
        cu = d["cu_seqlens"]
        for s in range(len(lengths)):
            sl = slice(int(cu[s]), int(cu[s + 1]))
            ys, hs = ssd.prefill(t["x"][sl], t["dt"][sl], t["A"], t["B"][sl], t["C"][sl], t["D"],
                                 t["h0"][s:s + 1].contiguous(), chunk=256)
            assert torch.equal(ys, y1[sl]) and torch.equal(hs[0], h1[s])
        hbuf = t["h0"].clone()
        y3, _ = ssd.prefill(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], hbuf, chunk=256,
                            cu_seqlens=t["cu_seqlens"], h_out=hbuf)
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
