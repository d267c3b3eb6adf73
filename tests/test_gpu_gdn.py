"""GPU gated delta rule (ssd_gated_delta_rule through the C ABI) against the
fp64 oracle (max-abs on every element of o and h_out: 1e-4 with float32
operands, 2e-2 with bfloat16 operands; the arithmetic is float32 in both)."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, log, maxabs
from state_space_model_amd import inputs

pytestmark = pytest.mark.gpu


def _gpu(d, dtype, dense_nseq=None, h0=True):
    import torch
    from state_space_model_amd import ssd
    op = torch.bfloat16 if dtype == "bf16" else torch.float32
    t = lambda a, o=None: torch.from_numpy(np.ascontiguousarray(a)).to("cuda") if o is None \
        else torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(o)
    cu = None if dense_nseq else t(d["cu_seqlens"].astype(np.int32))
    hz = t(d["h0"]) if (h0 and d["h0"] is not None) else None
    o, ho = ssd.gated_delta_rule(t(d["q"], op), t(d["k"], op), t(d["v"], op), t(d["g"]),
                                 t(d["beta"]), hz, cu, nseq=dense_nseq)
    torch.cuda.synchronize()
    return o.cpu().numpy(), ho.cpu().numpy()


def _ref(d, h0=True):
    hz = d["h0"].astype(np.float64) if (h0 and d["h0"] is not None) else None
    return oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], hz, d["cu_seqlens"])


SMALL = [  # (lengths, H, G, K, V, h0)
    ([100], 2, 1, 64, 16, False),
    ([257, 3, 130], 4, 2, 128, 32, True),
    ([300], 3, 3, 256, 48, True),
    ([33, 0, 70], 6, 2, 64, 128, True),
    ([1000], 2, 2, 128, 128, True),
    ([1, 1, 40], 4, 1, 128, 16, True),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_gdn_small(dtype, case):
    lengths, H, G, K, V, h0 = SMALL[case]
    log(f"gdn small dtype={dtype} lengths={lengths} H={H} G={G} K={K} V={V} h0={h0}")
    d = inputs.gdn_inputs(lengths, H, G, K, V, 900 + case, dtype=dtype, h0=h0)
    o, ho = _gpu(d, dtype)
    ro, rh = _ref(d)
    eo, eh = maxabs(o, ro), maxabs(ho, rh)
    log(f"  max|do|={eo:.3g} max|dh|={eh:.3g} (max|o|={np.max(np.abs(ro)):.3g})")
    assert eo <= TOL[dtype] and eh <= TOL[dtype]


def test_gdn_layer_workload():
    """The layer shape (4096 tokens, 32 heads over 16 groups, K = V = 128,
    bf16), every element of o and h_out against the full oracle."""
    w = inputs.GDN_W
    log("gdn layer workload (4096 tokens, H 32, G 16, K = V = 128, bf16), full oracle")
    d = inputs.gdn_inputs([w["L"]] * w["batch"], w["H"], w["G"], w["K"], w["V"], 950,
                          dtype=w["dtype"])
    o, ho = _gpu(d, "bf16")
    ro, rh = _ref(d)
    eo, eh = maxabs(o, ro), maxabs(ho, rh)
    log(f"  max|do|={eo:.3g} max|dh|={eh:.3g} (max|o|={np.max(np.abs(ro)):.3g})")
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"]


def test_gdn_packed_dense_solo_split():
    """Packed sequences get the same bits as each alone and as a dense batch;
    a sequence split in two with the state handed on equals one call."""
    import torch
    from state_space_model_amd import ssd
    lengths, H, G, K, V = [200, 200, 200], 4, 2, 128, 64
    d = inputs.gdn_inputs(lengths, H, G, K, V, 960, dtype="bf16", h0=True)
    o, ho = _gpu(d, "bf16")
    od, hd = _gpu(d, "bf16", dense_nseq=3)
    assert np.array_equal(o, od) and np.array_equal(ho, hd)
    cu = d["cu_seqlens"]
    for s in range(3):
        sl = slice(int(cu[s]), int(cu[s + 1]))
        ds = dict(d, q=d["q"][sl], k=d["k"][sl], v=d["v"][sl], g=d["g"][sl], beta=d["beta"][sl],
                  h0=d["h0"][s:s + 1], cu_seqlens=np.array([0, 200]))
        os_, hs = _gpu(ds, "bf16")
        assert np.array_equal(os_, o[sl]) and np.array_equal(hs[0], ho[s])
    # split at token 77 of the first sequence
    d1 = dict(d, q=d["q"][:77], k=d["k"][:77], v=d["v"][:77], g=d["g"][:77],
              beta=d["beta"][:77], h0=d["h0"][:1], cu_seqlens=np.array([0, 77]))
    o1, h1 = _gpu(d1, "bf16")
    d2 = dict(d, q=d["q"][77:200], k=d["k"][77:200], v=d["v"][77:200], g=d["g"][77:200],
              beta=d["beta"][77:200], h0=h1, cu_seqlens=np.array([0, 123]))
    o2, h2 = _gpu(d2, "bf16")
    assert maxabs(np.concatenate([o1, o2]), o[:200]) <= 1e-5
    assert maxabs(h2[0], ho[0]) <= 1e-5
    torch.cuda.synchronize()


def test_gdn_empty_and_alias():
    import torch
    from state_space_model_amd import ssd
    d = inputs.gdn_inputs([0, 0], 2, 1, 64, 16, 970, dtype="f32", h0=True)
    o, ho = _gpu(d, "f32")
    assert o.size == 0 and np.array_equal(ho, d["h0"])
    d = inputs.gdn_inputs([90, 40], 2, 1, 64, 32, 971, dtype="f32", h0=True)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    args = (t(d["q"]), t(d["k"]), t(d["v"]), t(d["g"]), t(d["beta"]))
    cu = t(d["cu_seqlens"].astype(np.int32))
    o1, h1 = ssd.gated_delta_rule(*args, t(d["h0"]), cu)
    hb = t(d["h0"]).clone()
    o2, h2 = ssd.gated_delta_rule(*args, hb, cu, h_out=hb)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, hb)
    lib = ssd.load()
    rc = lib.ssd_gated_delta_rule(None, None, None, None, None, None, None, None, None, 1, 64, 2,
                                  1, 96, 16, 0, None)
    assert rc == -2 and b"key dim" in lib.ssd_last_error()
