"""ctypes binding over libssd.so (C ABI in include/ssd.h).

Argument marshalling only: shape/dtype/device checks, output and workspace
allocation with torch, and the current torch stream handle.  Every step of the
computation runs in the HIP library; if the library is missing this module
raises instead of computing anything itself.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssd.so")

SSD_F32, SSD_BF16, SSD_F16 = 0, 1, 2
STAGE_CHUNK_CUMSUM, STAGE_CHUNK_STATE, STAGE_STATE_PASS, STAGE_CHUNK_SCAN = 1, 2, 4, 8
STAGE_ALL = 15
VARIANT_SCAN_ROWS, VARIANT_SCAN_HEADS = 0x100, 0x200
VARIANT_STATE_CHUNKS, VARIANT_STATE_WALK = 0x400, 0x800
NOALLOC_SCRATCH_BYTES = 32 << 20   # SSD_NOALLOC_SCRATCH_BYTES in ssd.h
SCAN_VARIANTS = {"auto": 0, "rows": VARIANT_SCAN_ROWS, "heads": VARIANT_SCAN_HEADS}
STATE_VARIANTS = {"auto": 0, "chunks": VARIANT_STATE_CHUNKS, "walk": VARIANT_STATE_WALK}
ERRORS = {0: "SSD_OK", -1: "SSD_ERR_INVALID_ARG", -2: "SSD_ERR_UNSUPPORTED",
          -3: "SSD_ERR_WORKSPACE", -4: "SSD_ERR_HIP"}
EXPORTS = ("ssd_scan_prefill_workspace", "ssd_scan_prefill_plan", "ssd_scan_prefill",
           "ssd_scan_prefill_stages", "ssd_scan_prefill_noalloc",
           "ssd_step", "ssd_step_multi", "ssd_conv1d_step", "ssd_gated_rmsnorm",
           "ssd_decode_layer_step", "ssd_selective_scan_workspace", "ssd_selective_scan",
           "ssd_scan_prefill_backward_workspace", "ssd_scan_prefill_backward",
           "ssd_scan_prefill_train_forward", "ssd_scan_prefill_backward_saved",
           "ssd_gated_delta_rule", "ssd_gated_delta_rule_chunked_workspace",
           "ssd_gated_delta_rule_chunked", "ssd_last_error")

_lib = None


class SSDError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


def load(path=LIB_PATH):
    """Load libssd.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with state_space_model_amd/build.py")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz, u32 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t,
                             ctypes.c_uint)
    lib.ssd_scan_prefill_workspace.argtypes = [i64, i32, i32, i32, i32, i32, i32, i32]
    lib.ssd_scan_prefill_workspace.restype = sz
    lib.ssd_scan_prefill_plan.argtypes = [i64, i32, i32, i32, i32, i32, i32, i32, i32]
    lib.ssd_scan_prefill_plan.restype = u32
    pre = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, i32, i32, vp, sz,
           vp]
    lib.ssd_scan_prefill.argtypes = pre
    lib.ssd_scan_prefill.restype = i32
    lib.ssd_scan_prefill_stages.argtypes = [u32] + pre
    lib.ssd_scan_prefill_stages.restype = i32
    lib.ssd_scan_prefill_noalloc.argtypes = pre[:-3] + [vp]
    lib.ssd_scan_prefill_noalloc.restype = i32
    lib.ssd_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.ssd_step.restype = i32
    lib.ssd_step_multi.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                   vp]
    lib.ssd_step_multi.restype = i32
    f32 = ctypes.c_float
    lib.ssd_conv1d_step.argtypes = [vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, vp]
    lib.ssd_conv1d_step.restype = i32
    lib.ssd_gated_rmsnorm.argtypes = [vp, vp, vp, f32, vp, i32, i32, i32, vp]
    lib.ssd_gated_rmsnorm.restype = i32
    lib.ssd_decode_layer_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp,
                                          i32, i32, i32, i32, i32, i32, i32, vp]
    lib.ssd_decode_layer_step.restype = i32
    lib.ssd_selective_scan_workspace.argtypes = [i32, i32, i32, i32]
    lib.ssd_selective_scan_workspace.restype = sz
    lib.ssd_selective_scan.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                       vp, sz, vp]
    lib.ssd_selective_scan.restype = i32
    lib.ssd_scan_prefill_backward_workspace.argtypes = [i64, i32, i32, i32, i32, i32, i32, i32]
    lib.ssd_scan_prefill_backward_workspace.restype = sz
    lib.ssd_scan_prefill_backward.argtypes = [vp] * 17 + [i32, i64, i32, i32, i32, i32, i32, i32,
                                                          vp, sz, vp]
    lib.ssd_scan_prefill_backward.restype = i32
    lib.ssd_scan_prefill_backward_saved.argtypes = lib.ssd_scan_prefill_backward.argtypes
    lib.ssd_scan_prefill_backward_saved.restype = i32
    lib.ssd_scan_prefill_train_forward.argtypes = [vp] * 10 + [i32, i64, i32, i32, i32, i32, i32,
                                                               i32, vp, sz, vp]
    lib.ssd_scan_prefill_train_forward.restype = i32
    lib.ssd_gated_delta_rule.argtypes = [vp] * 9 + [i32, i64, i32, i32, i32, i32, i32, vp]
    lib.ssd_gated_delta_rule.restype = i32
    lib.ssd_gated_delta_rule_chunked_workspace.argtypes = [i64, i32, i32, i32, i32, i32]
    lib.ssd_gated_delta_rule_chunked_workspace.restype = sz
    lib.ssd_gated_delta_rule_chunked.argtypes = [vp] * 9 + [i32, i64, i32, i32, i32, i32, i32, vp,
                                                            sz, vp]
    lib.ssd_gated_delta_rule_chunked.restype = i32
    lib.ssd_last_error.argtypes = []
    lib.ssd_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc):
    if rc != 0:
        raise SSDError(rc, load().ssd_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    if t.dtype == torch.float32:
        return SSD_F32
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    raise TypeError(f"x/B/C must be float32 or bfloat16, got {t.dtype}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype=None, dev=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _shape(t, name, shape):
    """Reject a tensor whose shape is not exactly `shape` (the C ABI cannot
    check the size of a device buffer, so an undersized one would be written
    out of bounds)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")


def workspace_bytes(total_tokens, nseq, H, P, N, G, chunk, dtype=torch.bfloat16):
    code = SSD_BF16 if dtype == torch.bfloat16 else SSD_F32
    return int(load().ssd_scan_prefill_workspace(total_tokens, nseq, H, P, N, G, chunk, code))


def plan(total_tokens, nseq, H, P, N, G, chunk, dtype=torch.bfloat16, packed=False):
    """The kernels a prefill of these shapes runs: {"state": "chunks"|"walk",
    "scan": "rows"|"heads"}, or None for shapes the library refuses."""
    code = SSD_BF16 if dtype == torch.bfloat16 else SSD_F32
    v = int(load().ssd_scan_prefill_plan(total_tokens, nseq, H, P, N, G, chunk, code,
                                         int(bool(packed))))
    if v == 0:
        return None
    return {"state": "walk" if v & VARIANT_STATE_WALK else "chunks",
            "scan": "heads" if v & VARIANT_SCAN_HEADS else "rows"}


def alloc_workspace(total_tokens, nseq, H, P, N, G, chunk, dtype, device):
    n = workspace_bytes(total_tokens, nseq, H, P, N, G, chunk, dtype)
    if n == 0:
        raise SSDError(-2, "unsupported prefill shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def prefill(x, dt, A, B, C, D, h0=None, chunk=256, cu_seqlens=None, *, nseq=None, y=None,
            h_out=None, workspace=None, stages=STAGE_ALL, scan="auto", state="auto",
            prepare=False, noalloc=False):
    """Chunked SSD prefill.

    x [T,H,P] (or [b,L,H,P]), dt [T,H], A [H], B/C [T,G,N], D [H], h0
    [nseq,H,N,P] float32 or None, cu_seqlens int32 [nseq+1] or None (dense
    batch: ``nseq`` sequences of T/nseq tokens; a 4-d x gives nseq = b).
    ``scan``: "auto" (the library's choice), "rows" or "heads" forces the
    chunk-scan kernel (SSD_VARIANT_SCAN_*); ``state``: "auto", "chunks" or
    "walk" forces how the states are formed (SSD_VARIANT_STATE_*).
    Returns (y [T,H,P] float32, h_out [nseq,H,N,P] float32); with
    ``prepare=True`` nothing runs and (Prepared, y, h_out) is returned.
    ``noalloc=True`` calls ssd_scan_prefill_noalloc: the library's built-in
    scratch replaces the workspace (every stage, the library's kernel choice;
    shapes whose workspace exceeds NOALLOC_SCRATCH_BYTES are refused).
    """
    dense4 = x.dim() == 4
    if dense4:
        b, L, H, P = x.shape
        nseq = b if nseq is None else nseq
        x = x.reshape(b * L, H, P)
        dt = dt.reshape(b * L, H)
        B = B.reshape(b * L, *B.shape[-2:])
        C = C.reshape(b * L, *C.shape[-2:])
    T, H, P = x.shape
    G, N = B.shape[-2], B.shape[-1]
    dev = x.device
    _need(x, "x", dev=dev)
    code = _dtype_code(x)
    for t, n in ((B, "B"), (C, "C")):
        _need(t, n, x.dtype, dev)
    for t, n in ((dt, "dt"), (A, "A"), (D, "D")):
        _need(t, n, torch.float32, dev)
    if tuple(dt.shape) != (T, H) or tuple(A.shape) != (H,) or tuple(D.shape) != (H,):
        raise ValueError("dt must be [T,H], A and D [H]")
    if tuple(B.shape) != (T, G, N) or tuple(C.shape) != (T, G, N):
        raise ValueError("B and C must be [T,G,N]")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        nseq = cu_seqlens.numel() - 1
    elif nseq is None:
        nseq = 1
    if h0 is not None:
        _need(h0, "h0", torch.float32, dev)
        if tuple(h0.shape) != (nseq, H, N, P):
            raise ValueError(f"h0 must be [{nseq},{H},{N},{P}]")
    if y is None:
        y = torch.empty((T, H, P), dtype=torch.float32, device=dev)
    if h_out is None:
        h_out = torch.empty((nseq, H, N, P), dtype=torch.float32, device=dev)
    _need(y, "y", torch.float32, dev)
    _need(h_out, "h_out", torch.float32, dev)
    _shape(y, "y", (T, H, P))
    _shape(h_out, "h_out", (nseq, H, N, P))
    if noalloc:
        if workspace is not None or stages != STAGE_ALL or scan != "auto" or state != "auto":
            raise ValueError("noalloc runs every stage with the library's kernel choice and "
                             "its own scratch (no workspace, stages, scan or state)")
        lib = load()
        args = (_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(y),
                _ptr(h_out), _ptr(cu_seqlens), nseq, T, H, P, N, G, chunk, code)
        if prepare:
            keep = (x, dt, A, B, C, D, h0, y, h_out, cu_seqlens)
            return Prepared(lib.ssd_scan_prefill_noalloc, args, None, keep), y, h_out
        _check(lib.ssd_scan_prefill_noalloc(*args, _stream()))
        if dense4:
            y = y.reshape(nseq, T // nseq, H, P)
        return y, h_out
    if workspace is None:
        workspace = alloc_workspace(T, nseq, H, P, N, G, chunk, x.dtype, dev)
    _need(workspace, "workspace", torch.uint8, dev)
    if scan not in SCAN_VARIANTS:
        raise ValueError(f"scan must be one of {sorted(SCAN_VARIANTS)} (got {scan!r})")
    if state not in STATE_VARIANTS:
        raise ValueError(f"state must be one of {sorted(STATE_VARIANTS)} (got {state!r})")
    stages = stages | SCAN_VARIANTS[scan] | STATE_VARIANTS[state]
    lib = load()
    args = (_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(y),
            _ptr(h_out), _ptr(cu_seqlens), nseq, T, H, P, N, G, chunk, code, _ptr(workspace),
            workspace.numel())
    if prepare:
        keep = (x, dt, A, B, C, D, h0, y, h_out, cu_seqlens, workspace)
        return Prepared(lib.ssd_scan_prefill_stages, args, stages, keep), y, h_out
    _check(lib.ssd_scan_prefill_stages(stages, *args, _stream()))
    if dense4:
        y = y.reshape(nseq, T // nseq, H, P)
    return y, h_out


class Prepared:
    """A validated, pre-marshalled call of one entry point.

    Shapes, dtypes and pointers are checked once (by ``prefill``/``step``
    with ``prepare=True``); calling the object only passes the current
    stream and the stage mask.  The tensors must stay alive and unchanged in
    shape while the object is used.  Useful in tight loops and under HIP
    graph capture (the stream is read at call time).
    """

    def __init__(self, fn, args, stages=None, keep=()):
        self._fn = fn
        self._args = args
        self._stages = stages
        self._keep = keep   # tensors whose memory the pointers refer to

    def __call__(self, stages=None):
        """Run the call; ``stages`` (prefill only) replaces the stage bits,
        keeping the call's kernel-variant bits."""
        s = _stream()
        if self._stages is None:
            rc = self._fn(*self._args, s)
        else:
            st = self._stages if stages is None else \
                (stages & STAGE_ALL) | (self._stages & ~STAGE_ALL)
            rc = self._fn(st, *self._args, s)
        if rc != 0:
            _check(rc)


class TrainSaved:
    """What ``prefill_train`` leaves for ``prefill_backward(..., saved=...)``:
    the backward workspace holding the forward's chunk map, decays and
    states, and the shape it was made for."""

    def __init__(self, workspace, key):
        self.workspace = workspace
        self.key = key


def prefill_train(x, dt, A, B, C, D, h0=None, chunk=256, cu_seqlens=None, *, nseq=None,
                  y=None, h_out=None, prepare=False):
    """The forward of a training step: (y, h_out) as ``prefill`` computes them
    (bitwise in float32; in bfloat16 the chunk states are formed in split
    precision for the backward, so they are closer to the exact values), plus
    a ``TrainSaved`` that lets ``prefill_backward`` skip its forward
    recompute.  Packed [T,...] layout as ``prefill_backward``.  With
    ``prepare=True`` nothing runs and (Prepared, y, h_out, saved) is returned."""
    T, H, P = x.shape
    G, N = B.shape[-2], B.shape[-1]
    dev = x.device
    _need(x, "x", dev=dev)
    code = _dtype_code(x)
    for t, n in ((B, "B"), (C, "C")):
        _need(t, n, x.dtype, dev)
    for t, n in ((dt, "dt"), (A, "A"), (D, "D")):
        _need(t, n, torch.float32, dev)
    _shape(dt, "dt", (T, H))
    _shape(A, "A", (H,))
    _shape(D, "D", (H,))
    _shape(B, "B", (T, G, N))
    _shape(C, "C", (T, G, N))
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        nseq = cu_seqlens.numel() - 1
    elif nseq is None:
        nseq = 1
    if h0 is not None:
        _need(h0, "h0", torch.float32, dev)
        if tuple(h0.shape) != (nseq, H, N, P):
            raise ValueError(f"h0 must be [{nseq},{H},{N},{P}]")
    if y is None:
        y = torch.empty((T, H, P), dtype=torch.float32, device=dev)
    if h_out is None:
        h_out = torch.empty((nseq, H, N, P), dtype=torch.float32, device=dev)
    _need(y, "y", torch.float32, dev)
    _need(h_out, "h_out", torch.float32, dev)
    _shape(y, "y", (T, H, P))
    _shape(h_out, "h_out", (nseq, H, N, P))
    lib = load()
    n = int(lib.ssd_scan_prefill_backward_workspace(T, nseq, H, P, N, G, chunk, code))
    if n == 0:
        raise SSDError(-2, "unsupported prefill shape")
    workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    saved = TrainSaved(workspace, (T, nseq, H, P, N, G, chunk, code))
    args = (_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(y),
            _ptr(h_out), _ptr(cu_seqlens), nseq, T, H, P, N, G, chunk, code, _ptr(workspace),
            workspace.numel())
    if prepare:
        keep = (x, dt, A, B, C, D, h0, y, h_out, cu_seqlens, workspace)
        return Prepared(lib.ssd_scan_prefill_train_forward, args, None, keep), y, h_out, saved
    _check(lib.ssd_scan_prefill_train_forward(*args, _stream()))
    return y, h_out, saved


def prefill_backward(x, dt, A, B, C, D, dy, h0=None, dh_out=None, chunk=256, cu_seqlens=None,
                     *, nseq=None, workspace=None, saved=None, prepare=False):
    """Gradients of ``prefill`` for dL/dy = dy and dL/dh_out = dh_out.

    x, dt, A, B, C, D, h0, cu_seqlens, nseq, chunk as given to ``prefill``
    (packed [T,...] layout); dy [T,H,P] in x's dtype; dh_out [nseq,H,N,P]
    float32 or None.  ``saved``: the ``TrainSaved`` of a ``prefill_train`` on
    the same inputs -- the forward's states are then taken from it instead of
    recomputed (same result, bitwise).  Returns a dict of float32
    tensors dx [T,H,P], ddt [T,H], dA [H], dB/dC [T,G,N], dD [H],
    dh0 [nseq,H,N,P]; with ``prepare=True`` nothing runs and
    (Prepared, grads) is returned.
    """
    T, H, P = x.shape
    G, N = B.shape[-2], B.shape[-1]
    dev = x.device
    _need(x, "x", dev=dev)
    code = _dtype_code(x)
    for t, n in ((B, "B"), (C, "C"), (dy, "dy")):
        _need(t, n, x.dtype, dev)
    for t, n in ((dt, "dt"), (A, "A"), (D, "D")):
        _need(t, n, torch.float32, dev)
    if tuple(dt.shape) != (T, H) or tuple(A.shape) != (H,) or tuple(D.shape) != (H,):
        raise ValueError("dt must be [T,H], A and D [H]")
    if tuple(B.shape) != (T, G, N) or tuple(C.shape) != (T, G, N):
        raise ValueError("B and C must be [T,G,N]")
    if tuple(dy.shape) != (T, H, P):
        raise ValueError("dy must be [T,H,P]")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        nseq = cu_seqlens.numel() - 1
    elif nseq is None:
        nseq = 1
    for t, n in ((h0, "h0"), (dh_out, "dh_out")):
        if t is not None:
            _need(t, n, torch.float32, dev)
            if tuple(t.shape) != (nseq, H, N, P):
                raise ValueError(f"{n} must be [{nseq},{H},{N},{P}]")
    lib = load()
    fn = lib.ssd_scan_prefill_backward
    if saved is not None:
        if saved.key != (T, nseq, H, P, N, G, chunk, code):
            raise ValueError("saved forward was made for another shape, chunk or dtype")
        workspace = saved.workspace
        fn = lib.ssd_scan_prefill_backward_saved
    if workspace is None:
        n = int(lib.ssd_scan_prefill_backward_workspace(T, nseq, H, P, N, G, chunk, code))
        if n == 0:
            raise SSDError(-2, "unsupported prefill shape")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(dx=torch.empty((T, H, P), **f32), ddt=torch.empty((T, H), **f32),
             dA=torch.empty(H, **f32), dB=torch.empty((T, G, N), **f32),
             dC=torch.empty((T, G, N), **f32), dD=torch.empty(H, **f32),
             dh0=torch.empty((nseq, H, N, P), **f32))
    args = (_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(dy),
            _ptr(dh_out), _ptr(g["dx"]), _ptr(g["ddt"]), _ptr(g["dA"]), _ptr(g["dB"]),
            _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dh0"]), _ptr(cu_seqlens), nseq, T, H, P, N, G,
            chunk, code, _ptr(workspace), workspace.numel())
    if prepare:
        keep = (x, dt, A, B, C, D, h0, dy, dh_out, cu_seqlens, workspace, g)
        return Prepared(fn, args, None, keep), g
    _check(fn(*args, _stream()))
    return g


def gated_delta_rule(q, k, v, g, beta, h0=None, cu_seqlens=None, *, nseq=None, o=None,
                     h_out=None, form="auto", workspace=None, prepare=False):
    """Gated delta rule scan.  q, k [T,G,K]; v [T,H,V] (float32 or bfloat16,
    all the same); g, beta [T,H] float32; h0 [nseq,H,V,K] float32 or None;
    cu_seqlens int32 [nseq+1] or None (dense: ``nseq`` sequences of T/nseq).
    ``form``: "chunked" (chunks of 64 tokens on MFMA; K in {64,128}, V % 32
    == 0, V + K <= 256), "stream" (token by token, any supported shape), or
    "auto" (chunked where the shape allows).
    Returns (o [T,H,V] float32, h_out [nseq,H,V,K] float32); with
    ``prepare=True`` nothing runs and (Prepared, o, h_out) is returned."""
    T, G, K = q.shape
    H, V = v.shape[1], v.shape[2]
    dev = q.device
    _need(q, "q", dev=dev)
    code = _dtype_code(q)
    for t, n in ((k, "k"), (v, "v")):
        _need(t, n, q.dtype, dev)
    for t, n in ((g, "g"), (beta, "beta")):
        _need(t, n, torch.float32, dev)
    if tuple(k.shape) != (T, G, K) or v.shape[0] != T:
        raise ValueError("k must be [T,G,K] and v [T,H,V]")
    if tuple(g.shape) != (T, H) or tuple(beta.shape) != (T, H):
        raise ValueError("g and beta must be [T,H]")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        nseq = cu_seqlens.numel() - 1
    elif nseq is None:
        nseq = 1
    if h0 is not None:
        _need(h0, "h0", torch.float32, dev)
        if tuple(h0.shape) != (nseq, H, V, K):
            raise ValueError(f"h0 must be [{nseq},{H},{V},{K}]")
    if o is None:
        o = torch.empty((T, H, V), dtype=torch.float32, device=dev)
    if h_out is None:
        h_out = torch.empty((nseq, H, V, K), dtype=torch.float32, device=dev)
    _need(o, "o", torch.float32, dev)
    _need(h_out, "h_out", torch.float32, dev)
    _shape(o, "o", (T, H, V))
    _shape(h_out, "h_out", (nseq, H, V, K))
    lib = load()
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(h_out),
            _ptr(cu_seqlens), nseq, T, H, G, K, V, code)
    if form not in ("auto", "chunked", "stream"):
        raise ValueError(f"form must be auto, chunked or stream (got {form!r})")
    nws = int(lib.ssd_gated_delta_rule_chunked_workspace(T, nseq, H, K, V, code))
    if form == "chunked" and nws == 0:
        raise SSDError(-2, f"chunked gated delta rule does not support K={K} V={V}")
    fn = lib.ssd_gated_delta_rule
    if nws > 0 and form != "stream":
        if workspace is None:
            workspace = torch.empty(nws, dtype=torch.uint8, device=dev)
        _need(workspace, "workspace", torch.uint8, dev)
        args = args + (_ptr(workspace), workspace.numel())
        fn = lib.ssd_gated_delta_rule_chunked
    if prepare:
        keep = (q, k, v, g, beta, h0, o, h_out, cu_seqlens, workspace)
        return Prepared(fn, args, None, keep), o, h_out
    _check(fn(*args, _stream()))
    return o, h_out


def step(x, dt, A, B, C, D, h, y=None, prepare=False):
    """One decode token; h [b,H,N,P] float32 is updated in place.  Returns y [b,H,P]."""
    b, H, P = x.shape
    G, N = B.shape[-2], B.shape[-1]
    dev = x.device
    _need(x, "x", dev=dev)
    code = _dtype_code(x)
    for t, n in ((B, "B"), (C, "C")):
        _need(t, n, x.dtype, dev)
    for t, n in ((dt, "dt"), (A, "A"), (D, "D"), (h, "h")):
        _need(t, n, torch.float32, dev)
    if tuple(h.shape) != (b, H, N, P) or tuple(B.shape) != (b, G, N) or tuple(C.shape) != (b, G, N):
        raise ValueError("h must be [b,H,N,P], B/C [b,G,N]")
    if tuple(dt.shape) != (b, H):
        raise ValueError("dt must be [b,H]")
    _shape(A, "A", (H,))
    _shape(D, "D", (H,))
    if y is None:
        y = torch.empty((b, H, P), dtype=torch.float32, device=dev)
    _need(y, "y", torch.float32, dev)
    _shape(y, "y", (b, H, P))
    args = (_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h), _ptr(y), b, H, P, N,
            G, code)
    if prepare:
        return Prepared(load().ssd_step, args, keep=(x, dt, A, B, C, D, h, y)), y
    _check(load().ssd_step(*args, _stream()))
    return y


def step_multi(x, dt, A, B, C, D, h, y=None, prepare=False):
    """`steps` decode tokens in one launch; h [b,H,N,P] float32 is updated in
    place.  x [S,b,H,P], dt [S,b,H], B/C [S,b,G,N].  Returns y [S,b,H,P]."""
    S, b, H, P = x.shape
    G, N = B.shape[-2], B.shape[-1]
    dev = x.device
    _need(x, "x", dev=dev)
    code = _dtype_code(x)
    for t, n in ((B, "B"), (C, "C")):
        _need(t, n, x.dtype, dev)
    for t, n in ((dt, "dt"), (A, "A"), (D, "D"), (h, "h")):
        _need(t, n, torch.float32, dev)
    if tuple(h.shape) != (b, H, N, P) or tuple(B.shape) != (S, b, G, N) or \
            tuple(C.shape) != (S, b, G, N):
        raise ValueError("h must be [b,H,N,P], B/C [S,b,G,N]")
    if tuple(dt.shape) != (S, b, H):
        raise ValueError("dt must be [S,b,H]")
    _shape(A, "A", (H,))
    _shape(D, "D", (H,))
    if y is None:
        y = torch.empty((S, b, H, P), dtype=torch.float32, device=dev)
    _need(y, "y", torch.float32, dev)
    _shape(y, "y", (S, b, H, P))
    args = (_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h), _ptr(y), S, b, H, P,
            N, G, code)
    if prepare:
        return Prepared(load().ssd_step_multi, args, keep=(x, dt, A, B, C, D, h, y)), y
    _check(load().ssd_step_multi(*args, _stream()))
    return y


def conv1d_step(u, conv_state, w, bias=None, silu=True, out=None):
    """One token of the causal depthwise conv.  u [b,C] (float32 or bfloat16);
    conv_state [b,C,W] float32, rolled in place; w [C,W]; bias [C] or None.
    Returns out [b,C] in u's dtype."""
    b, C = u.shape
    W = w.shape[1]
    dev = u.device
    _need(u, "u", dev=dev)
    code = _dtype_code(u)
    for t, n in ((conv_state, "conv_state"), (w, "w")):
        _need(t, n, torch.float32, dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, dev)
    if tuple(conv_state.shape) != (b, C, W) or tuple(w.shape) != (C, W) or \
            (bias is not None and tuple(bias.shape) != (C,)):
        raise ValueError("conv_state must be [b,C,W], w [C,W], bias [C]")
    if out is None:
        out = torch.empty_like(u)
    _need(out, "out", u.dtype, dev)
    _shape(out, "out", (b, C))
    _check(load().ssd_conv1d_step(_ptr(u), _ptr(conv_state), _ptr(w), _ptr(bias), int(bool(silu)),
                                  _ptr(out), b, C, W, code, _stream()))
    return out


def gated_rmsnorm(y, z, w, eps=1e-5, out=None):
    """y [b,D] float32, z [b,D] (float32 or bfloat16), w [D]:
    y*silu(z) / sqrt(mean(.^2) + eps) * w.  Returns [b,D] float32."""
    b, D = y.shape
    dev = y.device
    _need(y, "y", torch.float32, dev)
    _need(z, "z", dev=dev)
    code = _dtype_code(z)
    _need(w, "w", torch.float32, dev)
    if tuple(z.shape) != (b, D) or tuple(w.shape) != (D,):
        raise ValueError("z must be [b,D], w [D]")
    if out is None:
        out = torch.empty_like(y)
    _need(out, "out", torch.float32, dev)
    _shape(out, "out", (b, D))
    _check(load().ssd_gated_rmsnorm(_ptr(y), _ptr(z), _ptr(w), float(eps), _ptr(out), b, D, code,
                                    _stream()))
    return out


def decode_layer_step(xbc, z, dt, A, D, conv_state, conv_w, conv_b, h, norm_w, eps=1e-5, *,
                      H, P, N, G, out=None, xbc_act=None, y=None, prepare=False):
    """The layer body around the scan for one token: conv1d step (+SiLU) over
    the x|B|C channels, the decode step, the gated RMS norm.  xbc [b, H*P+2*G*N],
    z [b, H*P], dt [b,H]; conv_state [b, H*P+2*G*N, W] and h [b,H,N,P] are
    updated in place.  Returns out [b, H*P] float32."""
    b, Cn = xbc.shape
    inner = H * P
    W = conv_w.shape[1]
    dev = xbc.device
    _need(xbc, "xbc", dev=dev)
    code = _dtype_code(xbc)
    _need(z, "z", xbc.dtype, dev)
    for t, n in ((dt, "dt"), (A, "A"), (D, "D"), (conv_state, "conv_state"),
                 (conv_w, "conv_w"), (h, "h"), (norm_w, "norm_w")):
        _need(t, n, torch.float32, dev)
    if conv_b is not None:
        _need(conv_b, "conv_b", torch.float32, dev)
    if Cn != inner + 2 * G * N or tuple(z.shape) != (b, inner) or tuple(dt.shape) != (b, H) or \
            tuple(conv_state.shape) != (b, Cn, W) or tuple(conv_w.shape) != (Cn, W) or \
            tuple(h.shape) != (b, H, N, P) or tuple(norm_w.shape) != (inner,):
        raise ValueError("inconsistent decode-layer shapes")
    if out is None:
        out = torch.empty((b, inner), dtype=torch.float32, device=dev)
    if xbc_act is None:
        xbc_act = torch.empty(xbc.shape, dtype=torch.float32, device=dev)
    if y is None:
        y = torch.empty((b, inner), dtype=torch.float32, device=dev)
    for t, n, dt_ in ((out, "out", torch.float32), (xbc_act, "xbc_act", torch.float32),
                      (y, "y", torch.float32)):
        _need(t, n, dt_, dev)
    _shape(out, "out", (b, inner))
    _shape(xbc_act, "xbc_act", (b, Cn))
    _shape(y, "y", (b, inner))
    _shape(A, "A", (H,))
    _shape(D, "D", (H,))
    if conv_b is not None:
        _shape(conv_b, "conv_b", (Cn,))
    args = (_ptr(xbc), _ptr(z), _ptr(dt), _ptr(A), _ptr(D), _ptr(conv_state), _ptr(conv_w),
            _ptr(conv_b), _ptr(h), _ptr(norm_w), float(eps), _ptr(out), _ptr(xbc_act), _ptr(y),
            b, H, P, N, G, W, code)
    if prepare:
        keep = (xbc, z, dt, A, D, conv_state, conv_w, conv_b, h, norm_w, out, xbc_act, y)
        return Prepared(load().ssd_decode_layer_step, args, keep=keep), out
    _check(load().ssd_decode_layer_step(*args, _stream()))
    return out


def selective_scan(x, dt, A, B, C, D, h0=None, *, y=None, h_out=None, workspace=None,
                   prepare=False):
    """Mamba-1 selective scan.  x, dt [b,L,d] and B, C [b,L,N] in float32,
    bfloat16 or float16; A [d,N], D [d] float32; h0 [b,d,N] float32 or None.
    Returns (y [b,L,d] float32, h_out [b,d,N] float32)."""
    b, L, d = x.shape
    N = A.shape[1]
    dev = x.device
    _need(x, "x", dev=dev)
    codes = {torch.float32: SSD_F32, torch.bfloat16: SSD_BF16, torch.float16: SSD_F16}
    if x.dtype not in codes:
        raise TypeError(f"x must be float32, bfloat16 or float16, got {x.dtype}")
    code = codes[x.dtype]
    for t, n in ((dt, "dt"), (B, "B"), (C, "C")):
        _need(t, n, x.dtype, dev)
    for t, n in ((A, "A"), (D, "D")):
        _need(t, n, torch.float32, dev)
    if tuple(dt.shape) != (b, L, d) or tuple(A.shape) != (d, N) or tuple(D.shape) != (d,) or \
            tuple(B.shape) != (b, L, N) or tuple(C.shape) != (b, L, N):
        raise ValueError("dt must be [b,L,d], A [d,N], D [d], B/C [b,L,N]")
    if h0 is not None:
        _need(h0, "h0", torch.float32, dev)
        if tuple(h0.shape) != (b, d, N):
            raise ValueError("h0 must be [b,d,N]")
    if y is None:
        y = torch.empty((b, L, d), dtype=torch.float32, device=dev)
    if h_out is None:
        h_out = torch.empty((b, d, N), dtype=torch.float32, device=dev)
    _need(y, "y", torch.float32, dev)
    _need(h_out, "h_out", torch.float32, dev)
    _shape(y, "y", (b, L, d))
    _shape(h_out, "h_out", (b, d, N))
    lib = load()
    if workspace is None:
        n = int(lib.ssd_selective_scan_workspace(b, L, d, N))
        if n == 0:
            raise SSDError(-2, "unsupported selective-scan shape")
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    args = (_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(y), _ptr(h_out),
            b, L, d, N, code, _ptr(workspace), workspace.numel())
    if prepare:
        keep = (x, dt, A, B, C, D, h0, y, h_out, workspace)
        return Prepared(lib.ssd_selective_scan, args, keep=keep), y, h_out
    _check(lib.ssd_selective_scan(*args, _stream()))
    return y, h_out
