"""ssd_scan_prefill_noalloc (the prefill with the library's built-in scratch in
place of a workspace) against ssd_scan_prefill with a caller workspace, both
through the C ABI: two calls in a row, the second on a smaller input, each
equal to the workspace entry point bit for bit (the same kernels run on the
same inputs) and within the oracle tolerance."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, dev_inputs, log, maxabs
from state_space_model_amd import inputs

pytestmark = pytest.mark.gpu


def _call(fn_name, t, chunk, nseq, with_ws):
    import torch
    from state_space_model_amd import ssd
    lib = ssd.load()
    T, H, P = t["x"].shape
    G, N = t["B"].shape[-2:]
    code = ssd.SSD_BF16 if t["x"].dtype == torch.bfloat16 else ssd.SSD_F32
    y = torch.full((T, H, P), float("nan"), dtype=torch.float32, device="cuda")
    ho = torch.full((nseq, H, N, P), float("nan"), dtype=torch.float32, device="cuda")
    p = ssd._ptr
    args = [p(t["x"]), p(t["dt"]), p(t["A"]), p(t["B"]), p(t["C"]), p(t["D"]), p(t["h0"]),
            p(y), p(ho), p(t.get("cu_seqlens")), nseq, T, H, P, N, G, chunk, code]
    ws = None
    if with_ws:
        ws = ssd.alloc_workspace(T, nseq, H, P, N, G, chunk, t["x"].dtype, "cuda")
        args += [p(ws), ws.numel()]
    rc = getattr(lib, fn_name)(*args, ssd._stream())
    assert rc == 0, (fn_name, rc, lib.ssd_last_error())
    torch.cuda.synchronize()
    return y.cpu().numpy(), ho.cpu().numpy()


def _case(name, d, dtype, chunk):
    from state_space_model_amd import ssd
    t = dev_inputs(d, dtype)
    nseq = d["cu_seqlens"].size - 1
    T, H, P = d["x"].shape
    G, N = d["B"].shape[-2:]
    need = ssd.workspace_bytes(T, nseq, H, P, N, G, chunk, t["x"].dtype)
    log(f"noalloc {name}: T={T} nseq={nseq} H={H} P={P} N={N} G={G} Q={chunk} dtype={dtype} "
        f"workspace={need} of {ssd.NOALLOC_SCRATCH_BYTES}")
    assert 0 < need <= ssd.NOALLOC_SCRATCH_BYTES
    y, ho = _call("ssd_scan_prefill_noalloc", t, chunk, nseq, with_ws=False)
    yw, how = _call("ssd_scan_prefill", t, chunk, nseq, with_ws=True)
    assert np.array_equal(y, yw) and np.array_equal(ho, how), \
        (maxabs(y, yw), maxabs(ho, how))
    return y, ho


def test_noalloc_two_calls_match_workspace_entry_point():
    """The 130M-layer prefill (4096 tokens, 24 heads, chunk 256, bfloat16),
    then a smaller packed batch of three sequences in float32 at chunk 64:
    each call equals ssd_scan_prefill with a workspace, and the oracle."""
    w = inputs.WORKLOADS[1]
    d1 = inputs.workload_inputs(1)
    y1, h1 = _case("130m layer", d1, w.dtype, w.chunk)
    h0 = d1["h0"].astype(np.float64) if d1.get("h0") is not None else None
    ry, rh = oracle.prefill(d1["x"], d1["dt"], d1["A"], d1["B"], d1["C"], d1["D"], h0,
                            d1["cu_seqlens"])
    ey, eh = maxabs(y1, ry), maxabs(h1, rh)
    log(f"  vs oracle: max|dy|={ey:.3g} max|dh|={eh:.3g}")
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]

    d2 = inputs.prefill_inputs(4, 32, 64, 2, [300, 0, 141], 901, dtype="f32", h0=True)
    y2, h2 = _case("small packed", d2, "f32", 64)
    ry, rh = oracle.prefill(d2["x"], d2["dt"], d2["A"], d2["B"], d2["C"], d2["D"],
                            d2["h0"].astype(np.float64), d2["cu_seqlens"])
    ey, eh = maxabs(y2, ry), maxabs(h2, rh)
    log(f"  vs oracle: max|dy|={ey:.3g} max|dh|={eh:.3g}")
    assert ey <= TOL["f32"] and eh <= TOL["f32"]


def test_noalloc_refuses_shapes_beyond_the_scratch():
    """A workspace larger than the built-in scratch is refused with
    SSD_ERR_WORKSPACE, and the call leaves its outputs alone."""
    import torch
    from state_space_model_amd import ssd
    lib = ssd.load()
    T, nseq, H, P, N, G, Q = 32768, 4, 80, 64, 128, 1, 256
    assert ssd.workspace_bytes(T, nseq, H, P, N, G, Q) > ssd.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, H, P), dtype=torch.bfloat16, device="cuda")
    dt = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    A = torch.zeros(H, dtype=torch.float32, device="cuda")
    B = torch.zeros((T, G, N), dtype=torch.bfloat16, device="cuda")
    y = torch.full((T, H, P), 7.0, dtype=torch.float32, device="cuda")
    p = ssd._ptr
    rc = lib.ssd_scan_prefill_noalloc(p(x), p(dt), p(A), p(B), p(B), p(A), None, p(y), None,
                                      None, nseq, T, H, P, N, G, Q, ssd.SSD_BF16, ssd._stream())
    assert rc == -3, rc   # SSD_ERR_WORKSPACE
    assert b"scratch" in lib.ssd_last_error()
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
