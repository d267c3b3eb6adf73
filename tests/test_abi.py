"""C-ABI library checks that need no GPU: it loads, exports every symbol the
header declares, sizes workspaces, and refuses bad arguments before any
launch (error paths only; no compute call is made here)."""
import ctypes
import os
import re

import pytest

from state_space_model_amd import ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_\w+)\s*\(", src)))


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(ssd.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ssd.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_workspace_size():
    lib = ssd.load()
    w = lib.ssd_scan_prefill_workspace
    n1 = w(4096, 1, 24, 64, 128, 1, 256, 1)
    nc = 16
    # S (float32) + H_in (bf16) per chunk and head, and s, dt, u per chunk, head and row
    expect_min = nc * 24 * 128 * 64 * (4 + 2) + 3 * nc * 24 * 256 * 4
    # bf16, P 64, N 128, chunk 256: the row-split scan's C.B^T fragments per
    # (chunk, group), 1 KB per (16-row tile, 32-row block)
    cbg = nc * 1 * (256 // 16) * (256 // 32) * 1024
    # and B of every (chunk, group) in MFMA fragment order for the state walk
    bfrag = nc * 1 * 256 * 128 * 2
    assert expect_min + cbg + bfrag <= n1 <= expect_min + cbg + bfrag + 8192
    # the C.B^T and B-fragment regions grow with the group count, not the head count
    n8 = w(4096, 1, 24, 64, 128, 8, 256, 1)
    assert n8 - n1 == 7 * (cbg + bfrag)
    n32 = w(4096, 1, 24, 64, 128, 1, 256, 0)             # float32: H_in in float32, no C.B^T
    expect32 = nc * 24 * 128 * 64 * (4 + 4) + 3 * nc * 24 * 256 * 4
    assert expect32 <= n32 <= expect32 + 8192
    assert w(4096, 1, 24, 64, 100, 1, 256, 1) == 0       # unsupported N
    assert w(4096, 1, 24, 64, 128, 1, 96, 1) == 0        # unsupported chunk
    assert w(4096, 1, 24, 64, 128, 1, 16, 1) == 0        # chunk 16 is refused
    assert w(4096, 1, 24, 64, 128, 5, 256, 1) == 0       # H % G != 0
    assert w(4096, 1, 8192, 128, 128, 1, 512, 1) == 0    # x rows past 32-bit tile offsets
    assert w(4096, 1, 8192, 16, 128, 8192, 512, 1) == 0  # B rows past 32-bit tile offsets
    assert w(-1, 1, 24, 64, 128, 1, 256, 1) == 0
    assert w(0, 1, 24, 64, 128, 1, 256, 1) > 0


def test_cbg_region_sized_by_groups():
    """The workspace holds the row split's C.B^T fragments for every (chunk,
    group) for bf16 with P 64, N 128 and chunk <= 256, and nothing else
    depends on G."""
    w = ssd.load().ssd_scan_prefill_workspace
    for T, nseq, H, P, N, G, Q, dt in [(4096, 1, 24, 64, 128, 1, 256, "bf16"),
                                       (4096, 1, 24, 64, 128, 1, 256, "f32"),
                                       (4096, 1, 24, 64, 64, 1, 256, "bf16"),
                                       (4096, 1, 24, 64, 128, 1, 512, "bf16"),
                                       (32768, 4, 80, 64, 128, 1, 256, "bf16"),
                                       (1000, 3, 128, 64, 128, 8, 64, "bf16"),
                                       (1000, 3, 128, 64, 128, 2, 32, "bf16")]:
        e = 2 if dt == "bf16" else 4
        nc = (T + nseq * (Q - 1)) // Q
        region = nc * G * (Q // 16) * (Q // 32) * 1024
        base = sum(-(-b // 256) * 256 for b in (16 * max(nc, 1), 4 * (nseq + 1),
                                                  4 * nc * H * Q, 4 * nc * H * Q, 4 * nc * H * Q,
                                                  4 * nc * H * N * P, e * nc * H * N * P))
        got = w(T, nseq, H, P, N, G, Q, 1 if dt == "bf16" else 0)
        has = dt == "bf16" and P == 64 and N == 128 and Q <= 256
        walk = dt == "bf16" and P == 64 and N == 128 and Q <= 256
        bfrag = nc * G * Q * N * 2
        assert got == base + (-(-region // 256) * 256 if has else 0) + \
            (-(-bfrag // 256) * 256 if walk else 0), (T, nseq, H, P, N, G, Q, dt)


def test_plan_query():
    """The planning query names the kernels a call runs: the state walk for a
    batch of at least 128 (sequence, head) chains (bf16, P 64, N 128,
    chunk <= 256; a packed batch by lists), the heads-streamed scan from 2048
    (chunk, head) units."""
    plan = ssd.plan
    assert plan(32768, 4, 80, 64, 128, 1, 256) == {"state": "walk", "scan": "heads"}
    assert plan(4096, 1, 24, 64, 128, 1, 256) == {"state": "chunks", "scan": "rows"}
    assert plan(32768, 4, 80, 64, 128, 1, 256, torch_f32()) == {"state": "chunks",
                                                                 "scan": "rows"}
    assert plan(32768, 4, 80, 64, 128, 1, 512) == {"state": "chunks", "scan": "rows"}
    assert plan(85952, 8, 80, 64, 128, 1, 64, packed=True) == {"state": "walk",
                                                                "scan": "heads"}
    assert plan(85952, 8, 80, 64, 128, 1, 512, packed=True) == {"state": "chunks",
                                                                 "scan": "rows"}
    assert plan(4000, 1, 80, 64, 128, 1, 256, packed=True) == {"state": "chunks",
                                                               "scan": "rows"}
    # 2^30 or more (chunk, head) positions (here 128 x 8388615): too many for
    # the walk by lists
    assert plan(2**28 - 1, 8, 128, 64, 128, 1, 32, packed=True)["state"] == "chunks"
    assert plan(2**26, 8, 128, 64, 128, 1, 32, packed=True)["state"] == "walk"
    assert plan(4096, 1, 24, 64, 100, 1, 256) is None


def torch_f32():
    import torch
    return torch.float32


def _prefill_rc(**kw):
    lib = ssd.load()
    a = dict(x=1, dt=1, A=1, B=1, C=1, D=1, h0=None, y=1, h_out=None, cu=None, nseq=1, T=64,
             H=4, P=16, N=16, G=1, chunk=64, dtype=0, ws=None, wsb=0)
    a.update(kw)
    p = lambda v: None if v is None else ctypes.c_void_p(v)
    rc = lib.ssd_scan_prefill(p(a["x"]), p(a["dt"]), p(a["A"]), p(a["B"]), p(a["C"]), p(a["D"]),
                              p(a["h0"]), p(a["y"]), p(a["h_out"]), p(a["cu"]), a["nseq"], a["T"],
                              a["H"], a["P"], a["N"], a["G"], a["chunk"], a["dtype"], p(a["ws"]),
                              a["wsb"], None)
    return rc, lib.ssd_last_error().decode()


def test_noalloc_limit_matches_the_header():
    m = re.search(r"#define\s+SSD_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)",
                  open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == ssd.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("kw,code,frag", [
    (dict(T=32768, nseq=4, H=80, P=64, N=128, chunk=256, dtype=1), -3, "scratch holds"),
    (dict(H=6, G=4), -1, "H % G"),
    (dict(chunk=16), -2, "use chunk 32"),
    (dict(x=None), -1, "null"),
])
def test_noalloc_rejects_before_touching_the_device(kw, code, frag):
    """The built-in-scratch prefill checks shapes and its size limit on the
    host, before the scratch address is looked up."""
    lib = ssd.load()
    a = dict(x=1, dt=1, A=1, B=1, C=1, D=1, y=1, nseq=1, T=64, H=4, P=16, N=16, G=1, chunk=64,
             dtype=0)
    a.update(kw)
    p = lambda v: None if v is None else ctypes.c_void_p(v)
    rc = lib.ssd_scan_prefill_noalloc(p(a["x"]), p(a["dt"]), p(a["A"]), p(a["B"]), p(a["C"]),
                                      p(a["D"]), None, p(a["y"]), None, None, a["nseq"], a["T"],
                                      a["H"], a["P"], a["N"], a["G"], a["chunk"], a["dtype"], None)
    msg = lib.ssd_last_error().decode()
    assert rc == code and frag in msg, (rc, msg)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(H=6, G=4), -1, "H % G"),
    (dict(P=24), -2, "headdim"),
    (dict(N=100), -2, "d_state"),
    (dict(chunk=48), -2, "chunk"),
    (dict(chunk=16), -2, "use chunk 32"),
    (dict(chunk=1024), -2, "chunk"),
    (dict(H=8192, P=128, chunk=512), -2, "row stride"),  # 32-bit tile offsets
    (dict(nseq=0), -1, "nseq"),
    (dict(T=65, nseq=2), -1, "divisible"),
    (dict(x=None), -1, "null"),
    (dict(A=None), -1, "null"),
    (dict(dtype=7), -1, "dtype"),
    (dict(ws=None, wsb=0), -3, "workspace"),
    (dict(ws=256, wsb=16), -3, "workspace"),
])
def test_prefill_rejects_before_launch(kw, code, frag):
    rc, msg = _prefill_rc(**kw)
    assert rc == code and frag in msg, (rc, msg)


@pytest.mark.parametrize("stages,frag", [(16, "stage"), (0x1000, "stage"),
                                          (0x30f, "exclusive"), (0xc0f, "exclusive")])
def test_stage_mask_rejected(stages, frag):
    lib = ssd.load()
    rc = lib.ssd_scan_prefill_stages(stages, *([ctypes.c_void_p(1)] * 10), 1, 64, 4, 16, 16, 1,
                                     64, 0, ctypes.c_void_p(256), 1 << 30, None)
    assert rc == -1 and frag in lib.ssd_last_error().decode()


def test_variant_bits_match_the_header():
    src = open(HEADER).read()
    vals = {k: int(v, 16) for k, v in re.findall(r"(SSD_VARIANT_\w+)\s*=\s*(0x[0-9a-fA-F]+)u", src)}
    assert vals["SSD_VARIANT_SCAN_ROWS"] == ssd.VARIANT_SCAN_ROWS
    assert vals["SSD_VARIANT_SCAN_HEADS"] == ssd.VARIANT_SCAN_HEADS
    assert vals["SSD_VARIANT_STATE_CHUNKS"] == ssd.VARIANT_STATE_CHUNKS
    assert vals["SSD_VARIANT_STATE_WALK"] == ssd.VARIANT_STATE_WALK


@pytest.mark.parametrize("kw,code,frag", [
    (dict(H=6, G=4), -1, "H % G"),
    (dict(P=8), -2, "headdim"),
    (dict(N=0), -2, "d_state"),
    (dict(N=2048), -2, "d_state"),
    (dict(batch=-1), -1, "batch"),
    (dict(x=None), -1, "null"),
    (dict(dtype=3), -1, "dtype"),
])
def test_step_rejects_before_launch(kw, code, frag):
    lib = ssd.load()
    a = dict(x=1, batch=2, H=4, P=16, N=16, G=1, dtype=0)
    a.update(kw)
    p = ctypes.c_void_p
    xptr = None if a["x"] is None else p(a["x"])
    rc = lib.ssd_step(xptr, p(1), p(1), p(1), p(1), p(1), p(1), p(1), a["batch"], a["H"], a["P"],
                      a["N"], a["G"], a["dtype"], None)
    assert rc == code and frag in lib.ssd_last_error().decode()


@pytest.mark.parametrize("kw,code,frag", [
    (dict(H=6, G=4), -1, "H % G"),
    (dict(P=8), -2, "headdim"),
    (dict(N=48), -2, "d_state"),
    (dict(N=256), -2, "d_state"),
    (dict(steps=-1), -1, "steps"),
    (dict(batch=-1), -1, "batch"),
    (dict(x=None), -1, "null"),
    (dict(dtype=3), -1, "dtype"),
])
def test_step_multi_rejects_before_launch(kw, code, frag):
    lib = ssd.load()
    a = dict(x=1, steps=3, batch=2, H=4, P=16, N=16, G=1, dtype=0)
    a.update(kw)
    p = ctypes.c_void_p
    xptr = None if a["x"] is None else p(a["x"])
    rc = lib.ssd_step_multi(xptr, p(1), p(1), p(1), p(1), p(1), p(1), p(1), a["steps"], a["batch"],
                            a["H"], a["P"], a["N"], a["G"], a["dtype"], None)
    assert rc == code and frag in lib.ssd_last_error().decode()


@pytest.mark.parametrize("kw,code,frag", [
    (dict(N=3), -2, "d_state"),
    (dict(N=32), -2, "d_state"),
    (dict(dim=0), -1, "dim"),
    (dict(L=-1), -1, "L >= 0"),
    (dict(x=None), -1, "null"),
    (dict(dtype=5), -1, "dtype"),
    (dict(ws=0), -3, "workspace"),
])
def test_selective_scan_rejects_before_launch(kw, code, frag):
    lib = ssd.load()
    a = dict(x=1, batch=1, L=64, dim=8, N=4, dtype=2, ws=1 << 20)
    a.update(kw)
    p = ctypes.c_void_p
    xptr = None if a["x"] is None else p(a["x"])
    rc = lib.ssd_selective_scan(xptr, p(1), p(1), p(1), p(1), p(1), None, p(1), None, a["batch"],
                                a["L"], a["dim"], a["N"], a["dtype"], p(1), a["ws"], None)
    assert rc == code and frag in lib.ssd_last_error().decode()


def test_backward_workspace_size():
    lib = ssd.load()
    w = lib.ssd_scan_prefill_backward_workspace
    fwd = lib.ssd_scan_prefill_workspace(4096, 1, 24, 64, 128, 1, 256, 1)
    n1 = w(4096, 1, 24, 64, 128, 1, 256, 1)
    nc = 16
    # the forward's workspace, then: final states (f32), states entering each chunk
    # (f32), dH per chunk (bf16) and the part of it bf16 rounds away (bf16), the
    # <dH, H> partials, six per-row arrays, dA/dD partials, per-head dB and dC
    extra = (24 * 128 * 64 * 4 + nc * 24 * 128 * 64 * (4 + 2 + 2) + nc * 24 * 128 * 4
             + 6 * nc * 24 * 256 * 4 + 2 * nc * 24 * 4 + 2 * 4096 * 24 * 128 * 4)
    assert fwd + extra <= n1 <= fwd + extra + 16 * 256
    assert w(4096, 1, 24, 64, 128, 24, 256, 1) < n1       # H == G: no per-head dB/dC
    assert w(4096, 1, 24, 64, 128, 5, 256, 1) == 0        # H % G != 0
    assert w(4096, 1, 24, 64, 100, 1, 256, 1) == 0        # unsupported N
    assert w(0, 1, 24, 64, 128, 1, 256, 1) > 0


def _backward_rc(**kw):
    lib = ssd.load()
    a = dict(x=1, dy=1, ddt=1, dA=1, dB=1, dC=1, dD=1, nseq=1, T=64, H=4, P=16, N=16, G=1,
             chunk=64, dtype=0, ws=None, wsb=0)
    a.update(kw)
    p = lambda v: None if v is None else ctypes.c_void_p(v)
    one = p(1)
    rc = lib.ssd_scan_prefill_backward(p(a["x"]), one, one, one, one, one, None,
                                       p(a["dy"]), None, one, p(a["ddt"]), p(a["dA"]), p(a["dB"]),
                                       p(a["dC"]), p(a["dD"]), None, None, a["nseq"], a["T"],
                                       a["H"], a["P"], a["N"], a["G"], a["chunk"], a["dtype"],
                                       p(a["ws"]), a["wsb"], None)
    return rc, lib.ssd_last_error().decode()


@pytest.mark.parametrize("kw,code,frag", [
    (dict(H=6, G=4), -1, "H % G"),
    (dict(P=24), -2, "headdim"),
    (dict(N=100), -2, "d_state"),
    (dict(chunk=48), -2, "chunk"),
    (dict(x=None), -1, "null"),
    (dict(dy=None), -1, "null"),
    (dict(dA=None), -1, "null"),
    (dict(dtype=2), -1, "dtype"),
    (dict(ws=None, wsb=0), -3, "workspace"),
    (dict(ws=256, wsb=16), -3, "workspace"),
])
def test_backward_rejects_before_launch(kw, code, frag):
    rc, msg = _backward_rc(**kw)
    assert rc == code and frag in msg, (rc, msg)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(K=96), -2, "key dim"),
    (dict(V=20), -2, "value dim"),
    (dict(V=2048), -2, "value dim"),
    (dict(H=6, G=4), -1, "H % G"),
    (dict(nseq=0), -1, "nseq"),
    (dict(T=65, nseq=2), -1, "divisible"),
    (dict(q=None), -1, "null"),
    (dict(dtype=2), -1, "dtype"),
])
def test_gated_delta_rule_rejects_before_launch(kw, code, frag):
    lib = ssd.load()
    a = dict(q=1, nseq=1, T=64, H=4, G=2, K=128, V=64, dtype=0)
    a.update(kw)
    p = ctypes.c_void_p
    qp = None if a["q"] is None else p(a["q"])
    rc = lib.ssd_gated_delta_rule(qp, p(1), p(1), p(1), p(1), None, p(1), None, None, a["nseq"],
                                  a["T"], a["H"], a["G"], a["K"], a["V"], a["dtype"], None)
    assert rc == code and frag in lib.ssd_last_error().decode()


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(64, 4, 16)
    with pytest.raises(ValueError, match="GPU"):
        ssd.prefill(x, torch.zeros(64, 4), torch.zeros(4), torch.zeros(64, 1, 16),
                    torch.zeros(64, 1, 16), torch.zeros(4))


class _NoLib:
    """Stands in for libssd.so: any call into it fails the test (the binding
    must refuse bad shapes before calling the library)."""

    def __getattr__(self, name):
        raise AssertionError(f"library called ({name}) despite a bad argument")


@pytest.fixture
def no_device(monkeypatch):
    """Let CPU tensors pass the binding's device check, and make any library
    call an error, so the shape checks can be tested without a GPU."""
    import torch

    def need(t, name, dtype=None, dev=None):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")

    monkeypatch.setattr(ssd, "_need", need)
    monkeypatch.setattr(ssd, "load", lambda *a: _NoLib())


def _prefill_args(T=64, H=4, P=16, N=16, G=1):
    import torch
    f = torch.float32
    return (torch.zeros(T, H, P), torch.zeros(T, H, dtype=f), torch.zeros(H), torch.zeros(T, G, N),
            torch.zeros(T, G, N), torch.zeros(H))


@pytest.mark.parametrize("bad", ["y", "h_out", "A", "D", "dt", "B"])
def test_binding_rejects_wrong_prefill_shapes(no_device, bad):
    import torch
    x, dt, A, B, C, D = _prefill_args()
    kw = dict(y=torch.zeros(64, 4, 16), h_out=torch.zeros(1, 4, 16, 16),
              workspace=torch.zeros(1 << 16, dtype=torch.uint8))
    if bad == "y":
        kw["y"] = torch.zeros(63, 4, 16)
    elif bad == "h_out":
        kw["h_out"] = torch.zeros(1, 4, 16, 8)
    elif bad == "A":
        A = torch.zeros(3)
    elif bad == "D":
        D = torch.zeros(4, 1)
    elif bad == "dt":
        dt = torch.zeros(64, 3)
    elif bad == "B":
        B = torch.zeros(64, 1, 8)
    with pytest.raises(ValueError):
        ssd.prefill(x, dt, A, B, C, D, **kw)


@pytest.mark.parametrize("bad", ["y", "h_out"])
def test_binding_rejects_wrong_train_forward_shapes(no_device, bad):
    import torch
    x, dt, A, B, C, D = _prefill_args()
    kw = dict(y=torch.zeros(64, 4, 16), h_out=torch.zeros(1, 4, 16, 16))
    kw[bad] = torch.zeros(2, 4, 16, 16) if bad == "h_out" else torch.zeros(64, 4, 8)
    with pytest.raises(ValueError):
        ssd.prefill_train(x, dt, A, B, C, D, **kw)


@pytest.mark.parametrize("bad", ["y", "A", "D"])
@pytest.mark.parametrize("multi", [False, True])
def test_binding_rejects_wrong_step_shapes(no_device, bad, multi):
    import torch
    b, H, P, N, G, S = 2, 4, 16, 16, 1, 3
    lead = (S, b) if multi else (b,)
    x, dt = torch.zeros(*lead, H, P), torch.zeros(*lead, H)
    Bm, Cm = torch.zeros(*lead, G, N), torch.zeros(*lead, G, N)
    A, D, h = torch.zeros(H), torch.zeros(H), torch.zeros(b, H, N, P)
    y = torch.zeros(*lead, H, P)
    if bad == "y":
        y = torch.zeros(*lead, H, P - 1)
    elif bad == "A":
        A = torch.zeros(H + 1)
    else:
        D = torch.zeros(1)
    fn = ssd.step_multi if multi else ssd.step
    with pytest.raises(ValueError):
        fn(x, dt, A, Bm, Cm, D, h, y=y)


def test_binding_rejects_wrong_scan_variant(no_device):
    import torch
    x, dt, A, B, C, D = _prefill_args()
    with pytest.raises(ValueError, match="scan"):
        ssd.prefill(x, dt, A, B, C, D, y=torch.zeros(64, 4, 16),
                    h_out=torch.zeros(1, 4, 16, 16),
                    workspace=torch.zeros(1 << 16, dtype=torch.uint8), scan="diagonal")
