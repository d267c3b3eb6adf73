"""GPU Mamba-1 selective scan (ssd_selective_scan through the C ABI) against
the fp64 oracle."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, log, maxabs
from state_space_model_amd import inputs

pytestmark = pytest.mark.gpu

OPS = {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}


def _gpu(d, dtype, h0=True, **kw):
    import torch
    from state_space_model_amd import ssd
    op = getattr(torch, OPS[dtype])
    t = lambda a, o=None: torch.from_numpy(np.ascontiguousarray(a)).to("cuda") if o is None \
        else torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(o)
    hh = t(d["h0"]) if (h0 and d["h0"] is not None) else None
    y, ho = ssd.selective_scan(t(d["x"], op), t(d["dt"], op), t(d["A"]), t(d["B"], op),
                               t(d["C"], op), t(d["D"]), hh, **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy(), ho.cpu().numpy()


# The kernel computes in float32 from the same rounded inputs as the oracle,
# so the float32 bound applies to every operand dtype.
@pytest.mark.parametrize("b,L,dim,N,dtype,h0", [
    (1, 37, 5, 1, "f32", False), (2, 300, 70, 4, "bf16", True), (3, 1000, 33, 16, "f16", True),
    (1, 17, 300, 8, "f32", True), (2, 777, 257, 16, "bf16", False), (1, 513, 64, 2, "f16", True),
])
def test_selective_scan_small(b, L, dim, N, dtype, h0):
    log(f"selective scan b={b} L={L} dim={dim} N={N} dtype={dtype} h0={h0}")
    d = inputs.selective_scan_inputs(b, L, dim, N, 900 + L + dim, dtype, h0)
    y, ho = _gpu(d, dtype)
    ry, rh = oracle.selective_scan(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"])
    ey, eh = maxabs(y, ry), maxabs(ho, rh)
    log(f"  max|dy|={ey:.3g} max|dh|={eh:.3g}")
    assert ey <= TOL["f32"] and eh <= TOL["f32"]


def test_selective_scan_w1_shape():
    """The COREY W1 shape: batch 1, d_inner 1024, L 4096, d_state 16, float16,
    every output against the oracle."""
    w = inputs.S6_W1
    log("selective scan, W1 shape (1 x 4096 x 1024, N 16, f16)")
    d = inputs.selective_scan_inputs(w["batch"], w["L"], w["dim"], w["N"], 1100, w["dtype"])
    y, ho = _gpu(d, w["dtype"])
    ry, rh = oracle.selective_scan(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], None)
    ey, eh = maxabs(y, ry), maxabs(ho, rh)
    log(f"  max|dy|={ey:.3g} max|dh|={eh:.3g}")
    assert ey <= TOL["f32"] and eh <= TOL["f32"]


def test_selective_scan_split_empty_alias():
    """Two calls handing the state on equal one call; L = 0 copies h0 to h_out;
    h_out may be the h0 buffer."""
    import torch
    from state_space_model_amd import ssd
    d = inputs.selective_scan_inputs(2, 400, 40, 16, 1200, "f32", True)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    x, dt, A, B, C, D, h0 = (t(d[k]) for k in ("x", "dt", "A", "B", "C", "D", "h0"))
    y, h = ssd.selective_scan(x, dt, A, B, C, D, h0)
    k = 157
    y1, h1 = ssd.selective_scan(x[:, :k].contiguous(), dt[:, :k].contiguous(), A,
                                B[:, :k].contiguous(), C[:, :k].contiguous(), D, h0)
    y2, h2 = ssd.selective_scan(x[:, k:].contiguous(), dt[:, k:].contiguous(), A,
                                B[:, k:].contiguous(), C[:, k:].contiguous(), D, h1)
    torch.cuda.synchronize()
    assert maxabs(torch.cat([y1, y2], 1).cpu(), y.cpu()) <= TOL["f32"]
    assert maxabs(h2.cpu(), h.cpu()) <= TOL["f32"]
    y0, h00 = ssd.selective_scan(x[:, :0].contiguous(), dt[:, :0].contiguous(), A,
                                 B[:, :0].contiguous(), C[:, :0].contiguous(), D, h0)
    torch.cuda.synchronize()
    assert y0.numel() == 0 and torch.equal(h00, h0)
    hb = h0.clone()
    y3, _ = ssd.selective_scan(x, dt, A, B, C, D, hb, h_out=hb)
    torch.cuda.synchronize()
    assert torch.equal(y3, y) and torch.equal(hb, h)
