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


def test_graph_backward_and_delta_rule_replays_equal_eager():
    """Forward + backward of the prefill and a delta-rule scan in one HIP graph
    (the backward's reductions are fixed-order, so replays are bitwise equal)."""
    import torch
    from state_space_model_amd import ssd
    log("graph: prefill forward + backward (varlen, bf16, 4 heads in 2 groups) + delta rule, "
        "4 replays")
    d = inputs.prefill_inputs(4, 64, 64, 2, [300, 77], 33, dtype="bf16", h0=True)
    t = dev_inputs(d, "bf16")
    T = int(d["cu_seqlens"][-1])
    dy, dh = inputs.cotangents(T, 2, 4, 64, 64, 34, "bf16")
    dyt = torch.from_numpy(dy).cuda().to(torch.bfloat16)
    dht = torch.from_numpy(dh).cuda()
    args = (t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"])
    run_f, y, h = ssd.prefill(*args, t["h0"], chunk=64, cu_seqlens=t["cu_seqlens"], prepare=True)
    run_b, g = ssd.prefill_backward(*args, dyt, t["h0"], dht, chunk=64,
                                    cu_seqlens=t["cu_seqlens"], prepare=True)
    dg = inputs.gdn_inputs([90, 40], 4, 2, 128, 32, 35, dtype="bf16", h0=True)
    gt = lambda a, o=None: torch.from_numpy(np.ascontiguousarray(a)).cuda() if o is None \
        else torch.from_numpy(np.ascontiguousarray(a)).cuda().to(o)
    bf = torch.bfloat16
    run_g, o, ho = ssd.gated_delta_rule(gt(dg["q"], bf), gt(dg["k"], bf), gt(dg["v"], bf),
                                        gt(dg["g"]), gt(dg["beta"]), gt(dg["h0"]),
                                        gt(dg["cu_seqlens"].astype(np.int32)), prepare=True)
    outs = [y, h, o, ho] + [g[k] for k in sorted(g)]

    def once():
        run_f()
        run_b()
        run_g()

    once()
    torch.cuda.synchronize()
    ref = [a.clone() for a in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        once()
    for r in range(4):
        for a in outs:
            a.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(outs, ref)), r
        once()      # eager work between replays
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(outs, ref)), r


def test_graph_walk_and_noalloc_replays_equal_eager():
    """A dense batch large enough for the two-segment state walk (2 x 2048
    tokens, 64 heads, chunk 256: B fragments, walk, fix-up, heads-streamed or
    row-split scan) and a packed one walked by lists (3 ragged sequences, 64
    heads) through the workspace entry point, and a smaller packed batch
    through the no-allocation entry point, captured in one HIP graph: every
    replay equals the eager run bit for bit, with eager work between
    replays."""
    import torch
    from state_space_model_amd import ssd
    log("graph: two-segment walk, list walk and no-allocation prefills, 4 replays")
    d = inputs.prefill_inputs(64, 64, 128, 1, [2048, 2048], 77, dtype="bf16", h0=True)
    t = dev_inputs(d, "bf16")
    assert ssd.plan(4096, 2, 64, 64, 128, 1, 256)["state"] == "walk"
    run_w, y, h = ssd.prefill(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["h0"],
                              chunk=256, nseq=2, prepare=True)
    d3 = inputs.prefill_inputs(64, 64, 128, 1, [1500, 700, 2100], 79, dtype="bf16", h0=True)
    t3 = dev_inputs(d3, "bf16")
    assert ssd.plan(4300, 3, 64, 64, 128, 1, 256, packed=True)["state"] == "walk"
    run_l, y3, h3 = ssd.prefill(t3["x"], t3["dt"], t3["A"], t3["B"], t3["C"], t3["D"], t3["h0"],
                                chunk=256, cu_seqlens=t3["cu_seqlens"], prepare=True)
    d2 = inputs.prefill_inputs(4, 64, 128, 2, [300, 77], 78, dtype="bf16", h0=True)
    t2 = dev_inputs(d2, "bf16")
    run_n, y2, h2 = ssd.prefill(t2["x"], t2["dt"], t2["A"], t2["B"], t2["C"], t2["D"], t2["h0"],
                                chunk=64, cu_seqlens=t2["cu_seqlens"], noalloc=True,
                                prepare=True)

    def once():
        run_w()
        run_l()
        run_n()

    once()  # the first no-allocation call looks up the scratch address
    torch.cuda.synchronize()
    outs = (y, h, y3, h3, y2, h2)
    ref = [v.clone() for v in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        once()
    for r in range(4):
        for v in outs:
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for v, e in zip(outs, ref):
            assert torch.equal(v, e), r
        once()
        torch.cuda.synchronize()
        for v, e in zip(outs, ref):
            assert torch.equal(v, e), r
