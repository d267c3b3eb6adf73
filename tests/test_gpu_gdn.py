"""GPU gated delta rule through the C ABI, both forms -- token by token
(ssd_gated_delta_rule) and in chunks of 64 tokens on MFMA
(ssd_gated_delta_rule_chunked) -- against the fp64 oracle (max-abs on every
element of o and h_out: 1e-4 with float32 operands, 2e-2 with bfloat16
operands; the arithmetic is float32 in both)."""
import ctypes

import numpy as np
import pytest

import oracle
from gpu_util import TOL, log, maxabs
from state_space_model_amd import inputs

pytestmark = pytest.mark.gpu


FORMS = ["stream", "chunked"]


def _chunked_ok(K, V):
    return K in (64, 128) and V % 32 == 0 and V + K <= 256


def _gpu(d, dtype, dense_nseq=None, h0=True, form="stream"):
    import torch
    from state_space_model_amd import ssd
    op = torch.bfloat16 if dtype == "bf16" else torch.float32
    t = lambda a, o=None: torch.from_numpy(np.ascontiguousarray(a)).to("cuda") if o is None \
        else torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(o)
    cu = None if dense_nseq else t(d["cu_seqlens"].astype(np.int32))
    hz = t(d["h0"]) if (h0 and d["h0"] is not None) else None
    o, ho = ssd.gated_delta_rule(t(d["q"], op), t(d["k"], op), t(d["v"], op), t(d["g"]),
                                 t(d["beta"]), hz, cu, nseq=dense_nseq, form=form)
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
    ([150, 40], 2, 1, 64, 192, True),
    ([97], 4, 4, 128, 96, False),
]


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_gdn_small(dtype, case, form):
    lengths, H, G, K, V, h0 = SMALL[case]
    if form == "chunked" and not _chunked_ok(K, V):
        pytest.skip(f"chunked form: K={K} V={V} outside its shapes (the streaming form covers it)")
    log(f"gdn small form={form} dtype={dtype} lengths={lengths} H={H} G={G} K={K} V={V} h0={h0}")
    d = inputs.gdn_inputs(lengths, H, G, K, V, 900 + case, dtype=dtype, h0=h0)
    o, ho = _gpu(d, dtype, form=form)
    ro, rh = _ref(d)
    eo, eh = maxabs(o, ro), maxabs(ho, rh)
    log(f"  max|do|={eo:.3g} max|dh|={eh:.3g} (max|o|={np.max(np.abs(ro)):.3g})")
    assert eo <= TOL[dtype] and eh <= TOL[dtype]


@pytest.mark.parametrize("form", FORMS)
def test_gdn_layer_workload(form):
    """The layer shape (4096 tokens, 32 heads over 16 groups, K = V = 128,
    bf16), every element of o and h_out against the full oracle."""
    w = inputs.GDN_W
    log(f"gdn layer workload (4096 tokens, H 32, G 16, K = V = 128, bf16), {form}, full oracle")
    d = inputs.gdn_inputs([w["L"]] * w["batch"], w["H"], w["G"], w["K"], w["V"], 950,
                          dtype=w["dtype"])
    o, ho = _gpu(d, "bf16", form=form)
    ro, rh = _ref(d)
    eo, eh = maxabs(o, ro), maxabs(ho, rh)
    log(f"  max|do|={eo:.3g} max|dh|={eh:.3g} (max|o|={np.max(np.abs(ro)):.3g})")
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"]


@pytest.mark.parametrize("form", FORMS)
def test_gdn_packed_dense_solo_split(form):
    """Packed sequences get the same bits as each alone and as a dense batch;
    a sequence split in two with the state handed on equals one call (to
    float32 rounding token by token; the chunked form regroups the tokens of a
    split sequence into other chunks, so there to its bfloat16 operand
    rounding)."""
    import torch
    from state_space_model_amd import ssd
    lengths, H, G, K, V = [200, 200, 200], 4, 2, 128, 64
    d = inputs.gdn_inputs(lengths, H, G, K, V, 960, dtype="bf16", h0=True)
    o, ho = _gpu(d, "bf16", form=form)
    od, hd = _gpu(d, "bf16", dense_nseq=3, form=form)
    assert np.array_equal(o, od) and np.array_equal(ho, hd)
    cu = d["cu_seqlens"]
    for s in range(3):
        sl = slice(int(cu[s]), int(cu[s + 1]))
        ds = dict(d, q=d["q"][sl], k=d["k"][sl], v=d["v"][sl], g=d["g"][sl], beta=d["beta"][sl],
                  h0=d["h0"][s:s + 1], cu_seqlens=np.array([0, 200]))
        os_, hs = _gpu(ds, "bf16", form=form)
        assert np.array_equal(os_, o[sl]) and np.array_equal(hs[0], ho[s])
    # split at token 77 of the first sequence
    d1 = dict(d, q=d["q"][:77], k=d["k"][:77], v=d["v"][:77], g=d["g"][:77],
              beta=d["beta"][:77], h0=d["h0"][:1], cu_seqlens=np.array([0, 77]))
    o1, h1 = _gpu(d1, "bf16", form=form)
    d2 = dict(d, q=d["q"][77:200], k=d["k"][77:200], v=d["v"][77:200], g=d["g"][77:200],
              beta=d["beta"][77:200], h0=h1, cu_seqlens=np.array([0, 123]))
    o2, h2 = _gpu(d2, "bf16", form=form)
    tol = 1e-5 if form == "stream" else TOL["bf16"]
    eo, eh = maxabs(np.concatenate([o1, o2]), o[:200]), maxabs(h2[0], ho[0])
    log(f"  {form}: split vs one call max|do|={eo:.3g} max|dh|={eh:.3g}")
    assert eo <= tol and eh <= tol
    torch.cuda.synchronize()


@pytest.mark.parametrize("form", FORMS)
def test_gdn_empty_and_alias(form):
    import torch
    from state_space_model_amd import ssd
    d = inputs.gdn_inputs([0, 0], 2, 1, 64, 32, 970, dtype="f32", h0=True)
    o, ho = _gpu(d, "f32", form=form)
    assert o.size == 0 and np.array_equal(ho, d["h0"])
    d = inputs.gdn_inputs([90, 40], 2, 1, 64, 32, 971, dtype="f32", h0=True)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    args = (t(d["q"]), t(d["k"]), t(d["v"]), t(d["g"]), t(d["beta"]))
    cu = t(d["cu_seqlens"].astype(np.int32))
    o1, h1 = ssd.gated_delta_rule(*args, t(d["h0"]), cu, form=form)
    hb = t(d["h0"]).clone()
    o2, h2 = ssd.gated_delta_rule(*args, hb, cu, h_out=hb, form=form)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, hb)
    lib = ssd.load()
    rc = lib.ssd_gated_delta_rule(None, None, None, None, None, None, None, None, None, 1, 64, 2,
                                  1, 96, 16, 0, None)
    assert rc == -2 and b"key dim" in lib.ssd_last_error()


def test_gdn_chunked_equals_stream_and_rejects():
    """Both forms agree on a packed batch with ragged tails in float32 (to
    1e-4), and the chunked entry point refuses shapes it does not cover and a
    short workspace."""
    import torch
    from state_space_model_amd import ssd
    d = inputs.gdn_inputs([129, 64, 5, 300], 4, 2, 128, 64, 980, dtype="f32", h0=True)
    os_, hs = _gpu(d, "f32", form="stream")
    oc, hc = _gpu(d, "f32", form="chunked")
    log(f"  chunked vs stream: max|do|={maxabs(oc, os_):.3g} max|dh|={maxabs(hc, hs):.3g}")
    assert maxabs(oc, os_) <= 1e-4 and maxabs(hc, hs) <= 1e-4
    lib = ssd.load()
    assert lib.ssd_gated_delta_rule_chunked_workspace(100, 1, 2, 256, 64, 1) == 0
    assert lib.ssd_gated_delta_rule_chunked_workspace(100, 1, 2, 128, 136, 1) == 0
    n = lib.ssd_gated_delta_rule_chunked_workspace(100, 1, 2, 128, 64, 1)
    assert n > 0
    ws = torch.empty(n - 256, dtype=torch.uint8, device="cuda")
    z = torch.zeros(100 * 2 * 128, dtype=torch.bfloat16, device="cuda")
    f = torch.zeros(200, dtype=torch.float32, device="cuda")
    o = torch.empty(100 * 2 * 64, dtype=torch.float32, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = lib.ssd_gated_delta_rule_chunked(p(z), p(z), p(z), p(f), p(f), None, p(o), None, None,
                                          1, 100, 2, 1, 128, 64, 1, p(ws), ws.numel(), None)
    assert rc == -3 and b"workspace" in lib.ssd_last_error()
    rc = lib.ssd_gated_delta_rule_chunked(p(z), p(z), p(z), p(f), p(f), None, p(o), None, None,
                                          1, 100, 2, 1, 256, 64, 1, p(ws), ws.numel(), None)
    assert rc == -2


@pytest.mark.parametrize("form", FORMS)
def test_gdn_long_sequence(form):
    """One 16384-token sequence (256 chunks) with h0, 4 heads over 2 groups,
    K = V = 128, bf16: the chunked form's bfloat16-pair products must not let
    the error grow along the state's chain of chunks (every element of o and
    h_out against the full oracle)."""
    log(f"gdn long sequence (16384 tokens, H 4, G 2, K = V = 128, bf16), {form}")
    d = inputs.gdn_inputs([16384], 4, 2, 128, 128, 990, dtype="bf16", h0=True)
    o, ho = _gpu(d, "bf16", form=form)
    ro, rh = _ref(d)
    eo, eh = maxabs(o, ro), maxabs(ho, rh)
    tail = maxabs(o[-2048:], ro[-2048:])
    log(f"  max|do|={eo:.3g} (last 2048 tokens {tail:.3g}) max|dh|={eh:.3g} "
        f"(max|o|={np.max(np.abs(ro)):.3g})")
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"]
