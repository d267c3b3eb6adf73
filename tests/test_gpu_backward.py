"""GPU gradients of the chunked prefill (ssd_scan_prefill_backward through the
C ABI) against the fp64 reverse-mode oracle, plus invariants on the GPU.

Tolerance: every gradient array g is compared as
max|g_gpu - g_ref| / max(1, max|g_ref|) <= TOL[dtype] (1e-4 float32, 2e-2
bfloat16), the output tolerances of the forward applied relative to each
gradient's own scale (dB and dC sum over heads and tokens, so their scale
grows with the problem)."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, dev_inputs, log, maxabs
from state_space_model_amd import inputs

pytestmark = pytest.mark.gpu

GRADS = ("dx", "ddt", "dA", "dB", "dC", "dD", "dh0")


def scaled_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref)) / max(1.0, float(np.max(np.abs(ref)))))


def _gpu_bwd(d, dy, dh, dtype, chunk, with_h0=True, dense_nseq=None):
    import torch
    from state_space_model_amd import ssd
    t = dev_inputs(d, dtype)
    h0 = t["h0"] if with_h0 else None
    cu = None if dense_nseq else t["cu_seqlens"]
    dyt = torch.from_numpy(np.ascontiguousarray(dy)).to("cuda").to(t["x"].dtype)
    dht = None if dh is None else torch.from_numpy(np.ascontiguousarray(dh)).to("cuda")
    g = ssd.prefill_backward(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], dyt, h0, dht,
                             chunk=chunk, cu_seqlens=cu, nseq=dense_nseq)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in g.items()}


def _ref_bwd(d, dy, dh, with_h0=True):
    h0 = d["h0"].astype(np.float64) if (with_h0 and d.get("h0") is not None) else None
    return oracle.prefill_backward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], dy, h0, dh,
                                   d["cu_seqlens"])


# dA sums dt_i dz_i over every token of a head, and dz cancels heavily, so
# the bf16 layer workloads also hold it to a tighter bound than the others.
DA_TOL_BF16_LAYER = 5e-3


def _compare(g, r, tol, tight=None):
    errs = {k: scaled_err(g[k], r[k]) for k in GRADS}
    log("  " + " ".join(f"{k}={v:.2g}" for k, v in errs.items()))
    lim = {k: min(tol, (tight or {}).get(k, tol)) for k in GRADS}
    bad = {k: v for k, v in errs.items() if not v <= lim[k]}
    assert not bad, f"gradients over tolerance {lim}: {bad}"


SMALL = [  # (lengths, H, P, N, G, chunk, h0, dh_out)
    ([200], 4, 16, 16, 1, 64, False, False),
    ([300], 2, 32, 32, 1, 32, True, True),
    ([257, 3, 130], 4, 64, 128, 2, 64, True, True),
    ([1000], 3, 64, 64, 3, 128, True, False),
    ([520, 0, 77], 4, 128, 16, 4, 256, True, True),
    ([1100, 513], 2, 64, 128, 1, 512, True, True),
    ([96], 8, 16, 128, 8, 32, False, True),
    ([700, 1], 6, 64, 128, 2, 256, True, True),
    ([130, 45], 4, 64, 128, 2, 32, True, True),  # chunk 32: two-wave workgroups
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_backward_small(dtype, case):
    lengths, H, P, N, G, chunk, h0, dh_out = SMALL[case]
    log(f"backward small dtype={dtype} lengths={lengths} H={H} P={P} N={N} G={G} Q={chunk}"
        f" h0={h0} dh_out={dh_out}")
    d = inputs.prefill_inputs(H, P, N, G, lengths, 500 + case, dtype=dtype, h0=h0)
    dy, dh = inputs.cotangents(int(sum(lengths)), len(lengths), H, P, N, 600 + case, dtype,
                               dh_out)
    g = _gpu_bwd(d, dy, dh, dtype, chunk)
    r = _ref_bwd(d, dy, dh)
    _compare(g, r, TOL[dtype])


def test_backward_tiny_workload_f32():
    w = inputs.WORKLOADS[0]
    log("backward workload 0 (tiny, float32)")
    d = inputs.workload_inputs(0)
    T, nseq = int(d["cu_seqlens"][-1]), len(d["cu_seqlens"]) - 1
    dy, dh = inputs.cotangents(T, nseq, w.H, w.P, w.N, 700, "f32")
    _compare(_gpu_bwd(d, dy, dh, "f32", w.chunk), _ref_bwd(d, dy, dh), TOL["f32"])


def test_backward_130m_layer_workload():
    """The Mamba-2 130M layer shape (4096 tokens, 24 heads, bf16), every
    gradient element against the full oracle."""
    w = inputs.WORKLOADS[1]
    log("backward workload 1 (Mamba-2 130M layer, bf16), full oracle")
    d = inputs.workload_inputs(1)
    T, nseq = int(d["cu_seqlens"][-1]), len(d["cu_seqlens"]) - 1
    dy, dh = inputs.cotangents(T, nseq, w.H, w.P, w.N, 701, "bf16")
    r = _ref_bwd(d, dy, dh)
    g = _gpu_bwd(d, dy, dh, "bf16", w.chunk)
    _compare(g, r, TOL["bf16"], {"dA": DA_TOL_BF16_LAYER})


def test_backward_2p7b_layer_workload():
    """4 x 8192 tokens, 80 heads, h0 and dh_out given (bf16): the GPU runs the
    whole workload (20 heads of the group summed per DB/DC workgroup) and
    every gradient element is compared with one full oracle run."""
    w = inputs.WORKLOADS[2]
    log("backward workload 2 (Mamba-2 2.7B layer, bf16), every element")
    d = inputs.workload_inputs(2)
    T, nseq = int(d["cu_seqlens"][-1]), len(d["cu_seqlens"]) - 1
    dy, dh = inputs.cotangents(T, nseq, w.H, w.P, w.N, 702, "bf16")
    g = _gpu_bwd(d, dy, dh, "bf16", w.chunk)
    r = _ref_bwd(d, dy, dh)
    _compare(g, r, TOL["bf16"], {"dA": DA_TOL_BF16_LAYER})


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("nchunks,hb", [(7, 1), (300, 2), (500, 3), (800, 6)])
def test_backward_heads_per_block(dtype, nchunks, hb):
    """DB/DC with 1, 2, 3 or 6 heads of a group per workgroup (6 heads in one
    group, chunk 64), against the oracle.  The library takes the largest
    divisor of H/G that leaves at least 768 workgroups, so the chunk count
    picks hb: under 256 chunks one head per workgroup (partial rows per head),
    256-383 two, 384-767 three, from 768 the whole group on chip (no partial
    rows).  The last chunk of each run is ragged."""
    H, P, N, G, chunk = 6, 64, 64, 1, 64
    total = 64 * (nchunks - 1) + 13
    lengths = [total - total // 3, total // 3]
    log(f"backward heads per block={hb} (chunks ~{nchunks}) dtype={dtype} lengths={lengths}")
    d = inputs.prefill_inputs(H, P, N, G, lengths, 81, dtype=dtype, h0=True)
    dy, dh = inputs.cotangents(sum(lengths), 2, H, P, N, 82, dtype)
    g = _gpu_bwd(d, dy, dh, dtype, chunk)
    _compare(g, _ref_bwd(d, dy, dh), TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_deterministic_and_varlen_equals_solo(dtype):
    """Two runs give identical bits; each sequence of a packed batch gets the
    same per-token gradients as when run alone, and dA/dD are the sums."""
    import torch
    from state_space_model_amd import ssd
    lengths = [257, 3, 130, 0, 64]
    H, P, N, G, Q = 4, 64, 64, 2, 64
    d = inputs.prefill_inputs(H, P, N, G, lengths, 31, dtype=dtype, h0=True)
    dy, dh = inputs.cotangents(sum(lengths), len(lengths), H, P, N, 32, dtype)
    g1 = _gpu_bwd(d, dy, dh, dtype, Q)
    g2 = _gpu_bwd(d, dy, dh, dtype, Q)
    for k in GRADS:
        assert np.array_equal(g1[k], g2[k]), k
    cu = d["cu_seqlens"]
    dA = np.zeros(H)
    dD = np.zeros(H)
    for s, L in enumerate(lengths):
        sl = slice(int(cu[s]), int(cu[s + 1]))
        ds = dict(d, x=d["x"][sl], dt=d["dt"][sl], B=d["B"][sl], C=d["C"][sl],
                  h0=d["h0"][s:s + 1], cu_seqlens=np.array([0, L]))
        gs = _gpu_bwd(ds, dy[sl], dh[s:s + 1], dtype, Q)
        for k in ("dx", "ddt", "dB", "dC"):
            assert np.array_equal(gs[k], g1[k][sl]), (s, k)
        assert np.array_equal(gs["dh0"][0], g1["dh0"][s]), s
        dA += gs["dA"]
        dD += gs["dD"]
    assert scaled_err(g1["dA"], dA) <= 1e-5 and scaled_err(g1["dD"], dD) <= 1e-5
    torch.cuda.synchronize()


def test_backward_dense_equals_packed():
    """A dense batch (no cu_seqlens) gives the same bits as the same batch
    described by cu_seqlens."""
    lengths = [300, 300, 300]
    d = inputs.prefill_inputs(4, 64, 128, 1, lengths, 41, dtype="bf16", h0=True)
    dy, dh = inputs.cotangents(900, 3, 4, 64, 128, 42, "bf16")
    gp = _gpu_bwd(d, dy, dh, "bf16", 128)
    gd = _gpu_bwd(d, dy, dh, "bf16", 128, dense_nseq=3)
    for k in GRADS:
        assert np.array_equal(gp[k], gd[k]), k


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_chunk_invariant(dtype):
    d = inputs.prefill_inputs(4, 64, 64, 2, [700, 333], 51, dtype=dtype, h0=True)
    dy, dh = inputs.cotangents(1033, 2, 4, 64, 64, 52, dtype)
    base = _gpu_bwd(d, dy, dh, dtype, 64)
    for Q in (32, 128, 256, 512):
        g = _gpu_bwd(d, dy, dh, dtype, Q)
        errs = {k: scaled_err(g[k], base[k]) for k in GRADS}
        log(f"  Q={Q} vs 64: " + " ".join(f"{k}={v:.2g}" for k, v in errs.items()))
        assert all(v <= TOL[dtype] for v in errs.values()), (Q, errs)


def test_backward_split_hands_gradient_on():
    """A sequence cut in two: the second part's dh0 passed as the first part's
    dh_out gives the gradients of one call."""
    import torch
    from state_space_model_amd import ssd
    L, k, H, P, N = 1000, 377, 2, 64, 64
    d = inputs.prefill_inputs(H, P, N, 1, [L], 61, dtype="f32", h0=True)
    dy, dh = inputs.cotangents(L, 1, H, P, N, 62, "f32")
    full = _gpu_bwd(d, dy, dh, "f32", 128)
    t = dev_inputs(d, "f32")
    sl1, sl2 = slice(0, k), slice(k, L)
    _, hmid = ssd.prefill(t["x"][sl1], t["dt"][sl1], t["A"], t["B"][sl1], t["C"][sl1], t["D"],
                          t["h0"], chunk=128)
    torch.cuda.synchronize()
    part = lambda sl, h0: dict(d, x=d["x"][sl], dt=d["dt"][sl], B=d["B"][sl], C=d["C"][sl],
                               h0=h0, cu_seqlens=np.array([0, sl.stop - sl.start]))
    g2 = _gpu_bwd(part(sl2, hmid.cpu().numpy()), dy[sl2], dh, "f32", 128)
    g1 = _gpu_bwd(part(sl1, d["h0"]), dy[sl1], g2["dh0"], "f32", 128)
    for key in ("dx", "ddt", "dB", "dC"):
        assert scaled_err(np.concatenate([g1[key], g2[key]]), full[key]) <= TOL["f32"], key
    assert scaled_err(g1["dA"] + g2["dA"], full["dA"]) <= TOL["f32"]
    assert scaled_err(g1["dD"] + g2["dD"], full["dD"]) <= TOL["f32"]
    assert scaled_err(g1["dh0"], full["dh0"]) <= TOL["f32"]


def test_backward_empty_and_single_tokens():
    """No tokens: dA = dD = 0 and dh0 = dh_out, packed or dense; sequences of
    one token against the oracle."""
    import torch
    from state_space_model_amd import ssd
    H, P, N = 3, 32, 16
    for lengths, dense in (([0], False), ([0, 0], False), ([0], True)):
        log(f"  empty lengths={lengths} dense={dense}")
        d = inputs.prefill_inputs(H, P, N, 1, lengths, 71, dtype="f32", h0=True)
        dy, dh = inputs.cotangents(0, len(lengths), H, P, N, 72, "f32")
        g = _gpu_bwd(d, dy, dh, "f32", 64, dense_nseq=len(lengths) if dense else None)
        assert g["dx"].size == 0 and g["ddt"].size == 0 and g["dB"].size == 0
        assert np.all(g["dA"] == 0) and np.all(g["dD"] == 0)
        assert np.array_equal(g["dh0"], dh)
    d = inputs.prefill_inputs(H, P, N, 1, [1, 1, 1], 73, dtype="f32", h0=True)
    dy, dh = inputs.cotangents(3, 3, H, P, N, 74, "f32")
    _compare(_gpu_bwd(d, dy, dh, "f32", 32), _ref_bwd(d, dy, dh), TOL["f32"])
    torch.cuda.synchronize()


TRAIN_CASES = [  # (lengths, H, P, N, G, chunk, h0, dh_out, dtype)
    ([4096], 24, 64, 128, 1, 256, False, False, "bf16"),
    ([700, 1, 0, 300], 4, 64, 128, 2, 128, True, True, "bf16"),
    ([513, 64], 6, 32, 64, 3, 64, True, False, "f32"),
    ([1100, 513], 2, 64, 128, 1, 512, True, True, "f32"),
    ([2048] * 4, 80, 64, 128, 1, 256, True, True, "bf16"),
]


@pytest.mark.parametrize("case", range(len(TRAIN_CASES)))
def test_train_forward_and_saved_backward_bitwise(case):
    """The backward that takes the training forward's saved states gives every
    gradient bitwise as the backward that recomputes them -- twice in a row on
    the same saved states (the backward leaves them intact).  In float32 the
    training forward's y and h_out are bitwise the plain prefill's; in
    bfloat16 it forms the chunk states from a two-part (rounded value and
    remainder) weighted x, so its y and h_out are checked against the oracle
    and must be at least as close to it as the plain prefill's."""
    import torch
    from state_space_model_amd import ssd
    lengths, H, P, N, G, chunk, h0, dh, dtype = TRAIN_CASES[case]
    log(f"train forward + saved backward: lengths={lengths} H={H} P={P} N={N} G={G} "
        f"Q={chunk} h0={h0} dh_out={dh} {dtype}")
    d = inputs.prefill_inputs(H, P, N, G, lengths, 1300 + case, dtype=dtype, h0=h0)
    t = dev_inputs(d, dtype)
    T, nseq = int(d["cu_seqlens"][-1]), len(lengths)
    dy, dhv = inputs.cotangents(T, nseq, H, P, N, 1400 + case, dtype, dh)
    dyt = torch.from_numpy(dy).cuda().to(t["x"].dtype)
    dht = None if dhv is None else torch.from_numpy(dhv).cuda()
    fwd = (t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"])
    y1, h1 = ssd.prefill(*fwd, t["h0"], chunk=chunk, cu_seqlens=t["cu_seqlens"])
    y2, h2, saved = ssd.prefill_train(*fwd, t["h0"], chunk=chunk, cu_seqlens=t["cu_seqlens"])
    g1 = ssd.prefill_backward(*fwd, dyt, t["h0"], dht, chunk=chunk, cu_seqlens=t["cu_seqlens"])
    g2 = ssd.prefill_backward(*fwd, dyt, t["h0"], dht, chunk=chunk, cu_seqlens=t["cu_seqlens"],
                              saved=saved)
    g3 = ssd.prefill_backward(*fwd, dyt, t["h0"], dht, chunk=chunk, cu_seqlens=t["cu_seqlens"],
                              saved=saved)
    torch.cuda.synchronize()
    if dtype == "f32":
        assert torch.equal(y1, y2) and torch.equal(h1, h2)
    else:
        ry, rh = oracle.prefill(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"],
                                None if d.get("h0") is None else d["h0"].astype(np.float64),
                                d["cu_seqlens"])
        e1 = (maxabs(y1.cpu().numpy(), ry), maxabs(h1.cpu().numpy(), rh))
        e2 = (maxabs(y2.cpu().numpy(), ry), maxabs(h2.cpu().numpy(), rh))
        log(f"  vs oracle: prefill y {e1[0]:.3g} h {e1[1]:.3g}; training forward y {e2[0]:.3g}"
            f" h {e2[1]:.3g}")
        assert max(e2) <= TOL["bf16"]
        assert e2[1] <= 1.25 * e1[1] + 1e-6, (e1, e2)
    for k in GRADS:
        assert torch.equal(g1[k], g2[k]), k
        assert torch.equal(g1[k], g3[k]), k
    with pytest.raises(ValueError):
        ssd.prefill_backward(*fwd, dyt, t["h0"], dht, chunk=chunk * 2 if chunk < 512 else 64,
                             cu_seqlens=t["cu_seqlens"], saved=saved)
    log("  bitwise equal")
