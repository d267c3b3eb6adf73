"""fp64 CPU oracle for the Mamba-2 SSD recurrence (plain sequential definition).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  It never imports the
GPU package and the GPU package never imports it; the two share no code.

The arithmetic lives in ``ssd_oracle.c`` (the recurrence written out token by
token, in float64).  This module only marshals arrays through ctypes:

* ``prefill(x, dt, A, B, C, D, h0=None, cu_seqlens=None)`` -> ``(y, h_out)``
* ``step(x, dt, A, B, C, D, h)`` -> ``y`` (``h`` updated in place)
* ``prefill_backward(..., dy, dh_out)`` -> gradients of the prefill inputs
* ``gated_delta_rule(q, k, v, g, beta, h0=None, cu_seqlens=None)`` -> ``(o, h_out)``

Passages followed: COREY, section 3.1 (generic selective SSM update);
Compiler-First State Space Duality ..., Abstract (one scalar decay per head);
Mamba-2 SSD fused layer via VGpuWarp, "Lane mapping" (per-channel sweep over
d_state, one exp per step); Recurrence Scan, "One equation, one packed result"
(output and carried state both returned and both compared).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def load(path=None):
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = _bind(ctypes.CDLL(_build.LIB))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.ssd_ref_prefill.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, P, P, I]
    lib.ssd_ref_prefill.restype = I
    lib.ssd_ref_step.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I]
    lib.ssd_ref_conv1d_step.argtypes = [P, P, P, P, I, I, I, I, P]
    lib.ssd_ref_conv1d_step.restype = I
    lib.ssd_ref_gated_rmsnorm.argtypes = [P, P, P, ctypes.c_double, I, I, P]
    lib.ssd_ref_gated_rmsnorm.restype = I
    lib.ssd_ref_selective_scan.argtypes = [P, P, P, P, P, P, P, I, I, I, I, P, P, I]
    lib.ssd_ref_selective_scan.restype = I
    lib.ssd_ref_step.restype = I
    lib.ssd_ref_prefill_backward.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, P, P,
                                             P, P, P, P, P, P, P, I]
    lib.ssd_ref_prefill_backward.restype = I
    lib.ssd_ref_gated_delta_rule.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, P, P, I]
    lib.ssd_ref_gated_delta_rule.restype = I
    return lib


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads():
    """Threads for the oracle: the CPUs this process may use, at most
    OMP_NUM_THREADS (16 when unset)."""
    cap = int(os.environ.get("OMP_NUM_THREADS") or 16)
    return max(1, min(cap, len(os.sched_getaffinity(0))))


def prefill(x, dt, A, B, C, D, h0=None, cu_seqlens=None, threads=None, lib=None):
    """Sequential fp64 SSD over packed sequences.

    x [T,H,P], dt [T,H], A [H], B/C [T,G,N], D [H]; h0 [nseq,H,N,P] or None.
    cu_seqlens: int array [nseq+1] (None = one sequence of length T).
    A dense batch [b,L,...] may be passed flattened with
    ``cu_seqlens = arange(b+1)*L``.  Returns (y [T,H,P] f64, h_out [nseq,H,N,P] f64).
    """
    lib = lib or load()
    x, dt, A, B, C, D = (_f32(v) for v in (x, dt, A, B, C, D))
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    if cu_seqlens is None:
        cu_seqlens = np.array([0, T], dtype=np.int64)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    nseq = cu.shape[0] - 1
    assert cu[0] == 0 and cu[-1] == T
    assert dt.shape == (T, H) and A.shape == (H,) and D.shape == (H,)
    assert B.shape == (T, G, N) and C.shape == (T, G, N)
    h0c = None
    if h0 is not None:
        h0c = np.ascontiguousarray(np.asarray(h0, dtype=np.float64))
        assert h0c.shape == (nseq, H, N, P)
    y = np.empty((T, H, P), dtype=np.float64)
    h_out = np.empty((nseq, H, N, P), dtype=np.float64)
    rc = lib.ssd_ref_prefill(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                             _ptr(h0c), _ptr(cu), nseq, H, P, N, G, _ptr(y), _ptr(h_out),
                             threads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return y, h_out


def step(x, dt, A, B, C, D, h, threads=None, lib=None):
    """One fp64 decode token.  x [b,H,P], dt [b,H], B/C [b,G,N];
    h [b,H,N,P] float64, updated in place.  Returns y [b,H,P] f64."""
    lib = lib or load()
    x, dt, A, B, C, D = (_f32(v) for v in (x, dt, A, B, C, D))
    b, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    assert isinstance(h, np.ndarray) and h.dtype == np.float64 and h.flags.c_contiguous
    assert h.shape == (b, H, N, P)
    y = np.empty((b, H, P), dtype=np.float64)
    rc = lib.ssd_ref_step(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                          _ptr(h), _ptr(y), b, H, P, N, G, threads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return y


def conv1d_step(u, win, w, bias=None, silu=True, lib=None):
    """One token of the causal depthwise conv.  u [b,C]; win [b,C,W] float64,
    updated in place (oldest tap first); w [C,W]; bias [C] or None.
    Returns the output [b,C] f64 (after silu when ``silu``)."""
    lib = lib or load()
    u, w = _f32(u), _f32(w)
    bias = None if bias is None else _f32(bias)
    b, C = u.shape
    W = w.shape[1]
    assert isinstance(win, np.ndarray) and win.dtype == np.float64 and win.flags.c_contiguous
    assert win.shape == (b, C, W) and w.shape == (C, W)
    assert bias is None or bias.shape == (C,)
    out = np.empty((b, C), dtype=np.float64)
    rc = lib.ssd_ref_conv1d_step(_ptr(u), _ptr(win), _ptr(w), _ptr(bias), int(bool(silu)), b, C,
                                 W, _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def gated_rmsnorm(y, z, w, eps=1e-5, lib=None):
    """y [b,D] (float64), z [b,D], w [D]: y*silu(z) normalised by its root mean
    square over D (plus eps), times w.  Returns [b,D] f64."""
    lib = lib or load()
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float64))
    z, w = _f32(z), _f32(w)
    b, D = y.shape
    assert z.shape == (b, D) and w.shape == (D,)
    out = np.empty((b, D), dtype=np.float64)
    rc = lib.ssd_ref_gated_rmsnorm(_ptr(y), _ptr(z), _ptr(w), float(eps), b, D, _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def selective_scan(x, dt, A, B, C, D, h0=None, threads=None, lib=None):
    """Mamba-1 selective scan in fp64.  x, dt [b,L,d]; A [d,N]; B, C [b,L,N];
    D [d]; h0 [b,d,N] or None.  Returns (y [b,L,d] f64, h_out [b,d,N] f64)."""
    lib = lib or load()
    x, dt, A, B, C, D = (_f32(v) for v in (x, dt, A, B, C, D))
    b, L, d = x.shape
    N = A.shape[1]
    assert dt.shape == (b, L, d) and A.shape == (d, N) and D.shape == (d,)
    assert B.shape == (b, L, N) and C.shape == (b, L, N)
    h0c = None
    if h0 is not None:
        h0c = np.ascontiguousarray(np.asarray(h0, dtype=np.float64))
        assert h0c.shape == (b, d, N)
    y = np.empty((b, L, d), dtype=np.float64)
    h_out = np.empty((b, d, N), dtype=np.float64)
    rc = lib.ssd_ref_selective_scan(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                    _ptr(h0c), b, L, d, N, _ptr(y), _ptr(h_out),
                                    threads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return y, h_out


def prefill_backward(x, dt, A, B, C, D, dy, h0=None, dh_out=None, cu_seqlens=None, threads=None,
                     lib=None):
    """Reverse-mode gradients of ``prefill`` in fp64 for a loss with
    dL/dy = dy [T,H,P] and dL/dh_out = dh_out [nseq,H,N,P] (None = 0).
    Returns a dict with dx [T,H,P], ddt [T,H], dA [H], dB/dC [T,G,N], dD [H]
    and dh0 [nseq,H,N,P] (all float64)."""
    lib = lib or load()
    x, dt, A, B, C, D = (_f32(v) for v in (x, dt, A, B, C, D))
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    if cu_seqlens is None:
        cu_seqlens = np.array([0, T], dtype=np.int64)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    nseq = cu.shape[0] - 1
    assert cu[0] == 0 and cu[-1] == T
    assert dt.shape == (T, H) and A.shape == (H,) and D.shape == (H,)
    assert B.shape == (T, G, N) and C.shape == (T, G, N)
    f64 = lambda a: None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    h0c, dyc, dhc = f64(h0), f64(dy), f64(dh_out)
    assert dyc.shape == (T, H, P)
    assert h0c is None or h0c.shape == (nseq, H, N, P)
    assert dhc is None or dhc.shape == (nseq, H, N, P)
    out = dict(dx=np.empty((T, H, P)), ddt=np.empty((T, H)), dA=np.empty(H),
               dB=np.empty((T, G, N)), dC=np.empty((T, G, N)), dD=np.empty(H),
               dh0=np.empty((nseq, H, N, P)))
    rc = lib.ssd_ref_prefill_backward(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0c), _ptr(cu), nseq, H, P,
        N, G, _ptr(dyc), _ptr(dhc), _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA"]),
        _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dh0"]),
        threads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def gated_delta_rule(q, k, v, g, beta, h0=None, cu_seqlens=None, threads=None, lib=None):
    """Gated delta rule in fp64, token by token.  q, k [T,G,K]; v [T,H,V];
    g (log-gate, <= 0), beta [T,H]; h0 [nseq,H,V,K] or None; cu_seqlens
    [nseq+1] or None (one sequence).  Returns (o [T,H,V], h_out [nseq,H,V,K])."""
    lib = lib or load()
    q, k, v, g, beta = (_f32(a) for a in (q, k, v, g, beta))
    T, G, K = q.shape
    H, V = v.shape[1], v.shape[2]
    if cu_seqlens is None:
        cu_seqlens = np.array([0, T], dtype=np.int64)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    nseq = cu.shape[0] - 1
    assert cu[0] == 0 and cu[-1] == T
    assert k.shape == (T, G, K) and v.shape == (T, H, V)
    assert g.shape == (T, H) and beta.shape == (T, H)
    h0c = None
    if h0 is not None:
        h0c = np.ascontiguousarray(np.asarray(h0, dtype=np.float64))
        assert h0c.shape == (nseq, H, V, K)
    o = np.empty((T, H, V), dtype=np.float64)
    h_out = np.empty((nseq, H, V, K), dtype=np.float64)
    rc = lib.ssd_ref_gated_delta_rule(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0c),
                                      _ptr(cu), nseq, H, G, K, V, _ptr(o), _ptr(h_out),
                                      threads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return o, h_out
