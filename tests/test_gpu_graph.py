"""Prefill + decode captured in a HIP graph: every replay must equal the eager
result bit for bit (the library records no memset nodes; all buffers are
allocated before capture)."""
import numpy as np
import pytest

from gpu_util import dev_inputs, log
from state_space_model_amd import inputs

pytestmark = pytest.mark.gpu


def test_graph_replays_equal_eager():
    import torch
    from state_space_model_amd import ssd
    log("graph: prefill (varlen, bf16) + decode step, 4 replays")
    d = inputs.prefill_inputs(8, 64, 128, 2, [700, 301, 1024], 31, dtype="bf16", h0=True)
    t = dev_inputs(d, "bf16")
    h0 = t["h0"]
    run_p, y, h = ssd.prefill(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], h0, chunk=128,
                              cu_seqlens=t["cu_seqlens"], prepare=True)
    rng = np.random.Generator(np.random.PCG64(3))
    xd = torch.from_numpy(inputs.round_bf16(rng.standard_normal((3, 8, 64)).astype(np.float32))
                          ).cuda().to(torch.bfloat16)
    dtd = torch.from_numpy(d["dt"][:3].copy()).cuda()
    Bd = t["B"][:3].contiguous()
    Cd = t["C"][:3].contiguous()
    run_s, yd = ssd.step(xd, dtd, t["A"], Bd, Cd, t["D"], h, prepare=True)

    def once():
        run_p()
        run_s()

    once()
    torch.cuda.synchronize()
    ref = (y.clone(), h.clone(), yd.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        once()
    for r in range(4):
        y.zero_(), h.zero_(), yd.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref[0]) and torch.equal(h, ref[1]) and torch.equal(yd, ref[2]), r
        once()      # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y, ref[0]) and torch.equal(h, ref[1])
