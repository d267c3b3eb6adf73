"""GPU decode step (ssd_step through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, log, maxabs
from state_space_model_amd import inputs

pytestmark = pytest.mark.gpu


def _run_steps(d, dtype, steps):
    import torch
    from state_space_model_amd import ssd
    op = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = "cuda"
    h = torch.from_numpy(d["h"]).to(dev)
    A = torch.from_numpy(d["A"]).to(dev)
    D = torch.from_numpy(d["D"]).to(dev)
    x = torch.from_numpy(d["x"]).to(dev).to(op)
    dt = torch.from_numpy(d["dt"]).to(dev)
    B = torch.from_numpy(d["B"]).to(dev).to(op)
    C = torch.from_numpy(d["C"]).to(dev).to(op)
    ys = []
    for t in range(steps):
        ys.append(ssd.step(x[t].contiguous(), dt[t].contiguous(), A, B[t].contiguous(),
                           C[t].contiguous(), D, h))
    torch.cuda.synchronize()
    return np.stack([y.cpu().numpy() for y in ys]), h.cpu().numpy()


def _oracle_steps(d, steps, bsel=None):
    h = d["h"].astype(np.float64)
    sl = slice(None) if bsel is None else bsel
    h = np.ascontiguousarray(h[sl])
    ys = []
    for t in range(steps):
        ys.append(oracle.step(d["x"][t][sl], d["dt"][t][sl], d["A"], d["B"][t][sl], d["C"][t][sl],
                              d["D"], h))
    return np.stack(ys), h


def _small(b, H, P, N, G, steps, seed, dtype):
    rng = np.random.Generator(np.random.PCG64(seed))
    d = inputs.prefill_inputs(H, P, N, G, [b * steps], seed, dtype=dtype)
    lead = lambda a: np.ascontiguousarray(a.reshape(b, steps, *a.shape[1:]).swapaxes(0, 1))
    return dict(x=lead(d["x"]), dt=lead(d["dt"]), B=lead(d["B"]), C=lead(d["C"]), A=d["A"],
                D=d["D"], h=rng.normal(0, 0.1, size=(b, H, N, P)).astype(np.float32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("b,H,P,N,G", [(1, 1, 16, 16, 1), (3, 4, 32, 48, 2), (2, 8, 64, 128, 8),
                                       (5, 6, 128, 7, 3), (4, 2, 16, 1024, 1)])
def test_step_small(dtype, b, H, P, N, G):
    log(f"step small dtype={dtype} b={b} H={H} P={P} N={N} G={G}")
    d = _small(b, H, P, N, G, 5, 100 + b + H + P + N, dtype)
    y, h = _run_steps(d, dtype, 5)
    ry, rh = _oracle_steps(d, 5)
    assert maxabs(y, ry) <= TOL["f32"]
    assert maxabs(h, rh) <= TOL["f32"]


@pytest.fixture(scope="module")
def codestral_ref():
    """The Codestral decode workload's 128 steps through the fp64 oracle, every
    batch row and head (computed once for the module)."""
    d = inputs.workload_inputs(3)
    ry, rh = _oracle_steps(d, inputs.WORKLOADS[3].steps)
    return d, ry, rh


def test_step_codestral_workload(codestral_ref):
    """Full decode workload (b=64, H=128, P=64, N=128, G=8, 128 steps, float32):
    every element of every step's y and of the final state against the
    oracle."""
    w = inputs.WORKLOADS[3]
    log("step workload 3 (codestral decode), 128 steps, every element")
    d, ry, rh = codestral_ref
    y, h = _run_steps(d, "f32", w.steps)
    ey, eh = maxabs(y, ry), maxabs(h, rh)
    log(f"  max|dy|={ey:.3g} max|dh|={eh:.3g}")
    assert ey <= TOL["f32"] and eh <= TOL["f32"]


def test_step_batched_equals_solo():
    import torch
    from state_space_model_amd import ssd
    d = _small(6, 4, 64, 128, 2, 1, 7, "f32")
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    h = t(d["h"])
    y = ssd.step(t(d["x"][0]), t(d["dt"][0]), t(d["A"]), t(d["B"][0]), t(d["C"][0]), t(d["D"]), h)
    for i in range(6):
        hi = t(d["h"][i:i + 1])
        yi = ssd.step(t(d["x"][0][i:i + 1]), t(d["dt"][0][i:i + 1]), t(d["A"]),
                      t(d["B"][0][i:i + 1]), t(d["C"][0][i:i + 1]), t(d["D"]), hi)
        assert torch.equal(yi[0], y[i]) and torch.equal(hi[0], h[i])


def _run_multi(d, dtype, steps):
    import torch
    from state_space_model_amd import ssd
    op = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = "cuda"
    t = lambda a, o=None: torch.from_numpy(np.ascontiguousarray(a)).to(dev) if o is None \
        else torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(o)
    h = t(d["h"])
    y = ssd.step_multi(t(d["x"][:steps], op), t(d["dt"][:steps]), t(d["A"]),
                       t(d["B"][:steps], op), t(d["C"][:steps], op), t(d["D"]), h)
    torch.cuda.synchronize()
    return y.cpu().numpy(), h.cpu().numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("b,H,P,N,G,steps", [(1, 1, 16, 16, 1, 1), (3, 4, 32, 64, 2, 7),
                                             (2, 8, 64, 128, 8, 37), (5, 6, 128, 32, 3, 9),
                                             (2, 3, 16, 128, 1, 20), (1, 2, 128, 128, 2, 5)])
def test_step_multi_small(dtype, b, H, P, N, G, steps):
    """Many steps in one launch equal the fp64 oracle stepped token by token,
    and the same number of single-step launches on the GPU."""
    log(f"step_multi small dtype={dtype} b={b} H={H} P={P} N={N} G={G} steps={steps}")
    d = _small(b, H, P, N, G, steps, 300 + b + H + P + N + steps, dtype)
    y, h = _run_multi(d, dtype, steps)
    ry, rh = _oracle_steps(d, steps)
    ey, eh = maxabs(y, ry), maxabs(h, rh)
    ys, hs = _run_steps(d, dtype, steps)
    log(f"  vs oracle max|dy|={ey:.3g} max|dh|={eh:.3g}; vs single steps "
        f"{maxabs(y, ys):.3g} {maxabs(h, hs):.3g}")
    assert ey <= TOL["f32"] and eh <= TOL["f32"]
    assert maxabs(y, ys) <= 1e-5 and maxabs(h, hs) <= 1e-5


def test_step_multi_codestral_workload(codestral_ref):
    """The Codestral decode workload's 128 steps in one launch: every element
    against the oracle."""
    w = inputs.WORKLOADS[3]
    log("step_multi workload 3 (codestral decode), 128 steps in one launch, every element")
    d, ry, rh = codestral_ref
    y, h = _run_multi(d, "f32", w.steps)
    ey, eh = maxabs(y, ry), maxabs(h, rh)
    log(f"  max|dy|={ey:.3g} max|dh|={eh:.3g}")
    assert ey <= TOL["f32"] and eh <= TOL["f32"]


def test_step_multi_edge_cases():
    """Zero steps leave the state alone; a zero batch does nothing; bad shapes
    are refused before any launch."""
    import torch
    from state_space_model_amd import ssd
    d = _small(2, 2, 32, 16, 1, 3, 77, "f32")
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    h = t(d["h"])
    y = ssd.step_multi(t(d["x"][:0]), t(d["dt"][:0]), t(d["A"]), t(d["B"][:0]), t(d["C"][:0]),
                       t(d["D"]), h)
    torch.cuda.synchronize()
    assert y.numel() == 0 and np.array_equal(h.cpu().numpy(), d["h"])
    lib = ssd.load()
    rc = lib.ssd_step_multi(None, None, None, None, None, None, None, None, 1, 1, 2, 32, 100, 1,
                            0, None)
    assert rc == -2 and b"d_state" in lib.ssd_last_error()
