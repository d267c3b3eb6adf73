"""Independent fp64 numpy formulations used to pin the oracle.

None of these shares code with the oracle (C, sequential) or with the GPU
library.  Each is a different route to the same mathematics:

* ``unrolled``: the closed-form unrolling of the linear recurrence,
  h_t = (prod_{k<=t} a_k) h0 + sum_{s<=t} (prod_{s<k<=t} a_k) dt_s x_s (x) B_s,
  evaluated with explicit products, O(L^2).
* ``chunked``: the block (state space duality) evaluation with chunk size Q:
  a quadratic, causally masked form inside each chunk plus a chunk-to-chunk
  state carry.  This is the decomposition the GPU kernels implement
  (Compiler-First State Space Duality ..., Abstract: equal-length chunks whose
  work is dense contractions; Table 7: static lower-triangular mask; Recurrence
  Scan, "One equation, one packed result": chunks processed in order, the
  state left by one being the starting state of the next).
* ``prefix_sum_A0``: the A = 0 closed form (a cumulative sum).
Arrays: x [L,H,P], dt [L,H], A [H], B/C [L,G,N], D [H], h0 [H,N,P].
"""
import numpy as np


def _groups(H, G):
    return [(h * G) // H for h in range(H)]


def unrolled(x, dt, A, B, C, D, h0=None):
    x, dt, A, B, C, D = (np.asarray(v, np.float64) for v in (x, dt, A, B, C, D))
    L, H, P = x.shape
    N = B.shape[2]
    grp = _groups(H, B.shape[1])
    h0 = np.zeros((H, N, P)) if h0 is None else np.asarray(h0, np.float64)
    y = np.zeros((L, H, P))
    hs = np.zeros((L, H, N, P))
    for h in range(H):
        g = grp[h]
        a = np.exp(dt[:, h] * A[h])
        for t in range(L):
            st = np.prod(a[: t + 1]) * h0[h]
            for s in range(t + 1):
                st = st + np.prod(a[s + 1: t + 1]) * dt[s, h] * np.outer(B[s, g], x[s, h])
            hs[t, h] = st
            y[t, h] = C[t, g] @ st + D[h] * x[t, h]
    h_last = hs[-1] if L else h0
    return y, h_last


def chunked(x, dt, A, B, C, D, h0=None, Q=4):
    x, dt, A, B, C, D = (np.asarray(v, np.float64) for v in (x, dt, A, B, C, D))
    L, H, P = x.shape
    N = B.shape[2]
    grp = _groups(H, B.shape[1])
    h0 = np.zeros((H, N, P)) if h0 is None else np.asarray(h0, np.float64)
    y = np.zeros((L, H, P))
    h_out = np.zeros((H, N, P))
    for h in range(H):
        g = grp[h]
        Hc = h0[h].copy()
        for c0 in range(0, L, Q):
            sl = slice(c0, min(c0 + Q, L))
            Xc, dtc = x[sl, h], dt[sl, h]
            Bc, Cc = B[sl, g], C[sl, g]
            s = np.cumsum(dtc * A[h])                       # local cumulative log-decay
            seg = s[:, None] - s[None, :]
            mask = np.tril(np.ones_like(seg, dtype=bool))
            Lmat = np.where(mask, np.exp(np.where(mask, seg, 0.0)), 0.0)
            y_diag = ((Cc @ Bc.T) * Lmat * dtc[None, :]) @ Xc
            y_off = np.exp(s)[:, None] * (Cc @ Hc)
            y[sl, h] = y_diag + y_off + D[h] * Xc
            w = np.exp(s[-1] - s) * dtc                    # decay to the chunk end
            S = (Bc * w[:, None]).T @ Xc                   # [N,P] chunk state
            Hc = np.exp(s[-1]) * Hc + S
        h_out[h] = Hc
    return y, h_out


def prefix_sum_A0(x, dt, B, C, D, h0=None):
    x, dt, B, C, D = (np.asarray(v, np.float64) for v in (x, dt, B, C, D))
    L, H, P = x.shape
    N = B.shape[2]
    grp = _groups(H, B.shape[1])
    h0 = np.zeros((H, N, P)) if h0 is None else np.asarray(h0, np.float64)
    y = np.zeros((L, H, P))
    h_out = np.zeros((H, N, P))
    for h in range(H):
        g = grp[h]
        inc = dt[:, h, None, None] * B[:, g, :, None] * x[:, h, None, :]   # [L,N,P]
        hs = h0[h][None] + np.cumsum(inc, axis=0)
        y[:, h] = np.einsum("tn,tnp->tp", C[:, g], hs) + D[h] * x[:, h]
        h_out[h] = hs[-1] if L else h0[h]
    return y, h_out
