"""Seeded sweep over the supported shape space: for each draw (P, N, chunk, G,
H, ragged packed lengths including empty and one-token sequences, h0 and
dh_out on or off, dtype), the prefill, its gradients and the gated delta rule
are compared with the fp64 oracle on every element (tolerances as the other
GPU tests: max-abs 1e-4 / 2e-2 on y and h_out; gradients relative to their own
scale).  The draws are fixed by the seed, so a failure names its case."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, dev_inputs, log, maxabs
from state_space_model_amd import inputs

pytestmark = pytest.mark.gpu

N_CASES = 12


def _draw(i):
    rng = np.random.Generator(np.random.PCG64(7000 + i))
    P = int(rng.choice([16, 32, 64, 128]))
    N = int(rng.choice([16, 32, 64, 128]))
    Q = int(rng.choice([32, 64, 128, 256, 512]))
    G = int(rng.choice([1, 2, 4]))
    H = G * int(rng.choice([1, 2, 3]))
    nseq = int(rng.integers(1, 4))
    lengths = [int(v) for v in rng.choice([0, 1, 17, 63, 64, 65, 200, 511, 700], size=nseq)]
    if sum(lengths) == 0:
        lengths[0] = 33
    return dict(P=P, N=N, Q=Q, G=G, H=H, lengths=lengths, h0=bool(rng.integers(0, 2)),
                dh=bool(rng.integers(0, 2)), dtype="bf16" if rng.integers(0, 2) else "f32")


def _scaled(a, b):
    b = np.asarray(b, np.float64)
    return 0.0 if b.size == 0 else maxabs(a, b) / max(1.0, float(np.max(np.abs(b))))


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_prefill_and_backward(i):
    import torch
    from state_space_model_amd import ssd
    c = _draw(i)
    log(f"sweep {i}: {c}")
    d = inputs.prefill_inputs(c["H"], c["P"], c["N"], c["G"], c["lengths"], 7100 + i,
                              dtype=c["dtype"], h0=c["h0"])
    t = dev_inputs(d, c["dtype"])
    y, ho = ssd.prefill(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"], chunk=c["Q"],
                        cu_seqlens=t["cu_seqlens"])
    T, nseq = int(d["cu_seqlens"][-1]), len(c["lengths"])
    dy, dh = inputs.cotangents(T, nseq, c["H"], c["P"], c["N"], 7200 + i, c["dtype"], c["dh"])
    dyt = torch.from_numpy(dy).cuda().to(t["x"].dtype)
    dht = None if dh is None else torch.from_numpy(dh).cuda()
    g = ssd.prefill_backward(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], dyt, t["h0"], dht,
                             chunk=c["Q"], cu_seqlens=t["cu_seqlens"])
    torch.cuda.synchronize()
    h0 = None if d["h0"] is None else d["h0"].astype(np.float64)
    ry, rh = oracle.prefill(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], h0, d["cu_seqlens"])
    r = oracle.prefill_backward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], dy, h0, dh,
                                d["cu_seqlens"])
    ey, eh = maxabs(y.cpu().numpy(), ry), maxabs(ho.cpu().numpy(), rh)
    eg = {k: _scaled(g[k].cpu().numpy(), r[k]) for k in r}
    log(f"  y {ey:.2g} h {eh:.2g} " + " ".join(f"{k} {v:.2g}" for k, v in eg.items()))
    tol = TOL[c["dtype"]]
    assert ey <= tol and eh <= tol, (ey, eh)
    assert all(v <= tol for v in eg.values()), eg


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_gated_delta_rule(i):
    import torch
    from state_space_model_amd import ssd
    rng = np.random.Generator(np.random.PCG64(7300 + i))
    K = int(rng.choice([64, 128, 256]))
    V = 16 * int(rng.integers(1, 9))
    G = int(rng.choice([1, 2]))
    H = G * int(rng.choice([1, 2, 4]))
    lengths = [int(v) for v in rng.choice([0, 1, 31, 32, 33, 150], size=int(rng.integers(1, 4)))]
    dtype = "bf16" if rng.integers(0, 2) else "f32"
    h0 = bool(rng.integers(0, 2))
    log(f"gdn sweep {i}: K={K} V={V} H={H} G={G} lengths={lengths} dtype={dtype} h0={h0}")
    d = inputs.gdn_inputs(lengths, H, G, K, V, 7400 + i, dtype=dtype, h0=h0)
    op = torch.bfloat16 if dtype == "bf16" else torch.float32
    tt = lambda a, o=None: torch.from_numpy(np.ascontiguousarray(a)).cuda() if o is None \
        else torch.from_numpy(np.ascontiguousarray(a)).cuda().to(o)
    o, ho = ssd.gated_delta_rule(tt(d["q"], op), tt(d["k"], op), tt(d["v"], op), tt(d["g"]),
                                 tt(d["beta"]), None if d["h0"] is None else tt(d["h0"]),
                                 tt(d["cu_seqlens"].astype(np.int32)))
    torch.cuda.synchronize()
    hz = None if d["h0"] is None else d["h0"].astype(np.float64)
    ro, rh = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], hz,
                                     d["cu_seqlens"])
    eo, eh = maxabs(o.cpu().numpy(), ro), maxabs(ho.cpu().numpy(), rh)
    log(f"  o {eo:.2g} h {eh:.2g}")
    assert eo <= TOL[dtype] and eh <= TOL[dtype]
