"""Helpers for the GPU parity tests: upload seeded inputs, sample heads for
the oracle, compare.  Inputs come from state_space_model_amd.inputs; expected
values come only from the oracle."""
import sys

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}   # max-abs on every compared element of y and h_out


RECORD = []   # error figures of this session, printed in pytest's terminal summary


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()
    RECORD.append(msg)


def dev_inputs(d, dtype):
    import torch
    dev = "cuda"
    op = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {}
    for k in ("x", "B", "C"):
        out[k] = torch.from_numpy(np.ascontiguousarray(d[k])).to(dev).to(op).contiguous()
    for k in ("dt", "A", "D"):
        out[k] = torch.from_numpy(np.ascontiguousarray(d[k])).to(dev)
    if d.get("h0") is not None:
        out["h0"] = torch.from_numpy(np.ascontiguousarray(d["h0"])).to(dev)
    else:
        out["h0"] = None
    if "cu_seqlens" in d:
        out["cu_seqlens"] = torch.from_numpy(d["cu_seqlens"].astype(np.int32)).to(dev)
    return out


def select_heads(d, heads, G):
    """Inputs restricted to a subset of heads (each keeps its own B/C group)."""
    H = d["A"].shape[0]
    grp = [(h * G) // H for h in heads]
    out = dict(d)
    out["x"] = np.ascontiguousarray(d["x"][:, heads])
    out["dt"] = np.ascontiguousarray(d["dt"][:, heads])
    out["A"] = d["A"][heads]
    out["D"] = d["D"][heads]
    out["B"] = np.ascontiguousarray(d["B"][:, grp])
    out["C"] = np.ascontiguousarray(d["C"][:, grp])
    if d.get("h0") is not None:
        out["h0"] = np.ascontiguousarray(d["h0"][:, heads])
    return out


def maxabs(a, b, block=1 << 22):
    """max |a - b| over every element, in float64 (blockwise, so that large
    arrays need no full-size temporaries)."""
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, (a.shape, b.shape)
    fa, fb = a.reshape(-1), b.reshape(-1)
    m = 0.0
    for i in range(0, fa.size, block):
        d = np.abs(fa[i:i + block].astype(np.float64) - fb[i:i + block].astype(np.float64))
        m = max(m, float(np.max(d, initial=0.0)))
    return m


def ssm_scale(y_ref, x, D):
    """max |y_ref - D x|: the size of the state-space part of the output (the
    skip term D x dominates |y| at these distributions)."""
    T = y_ref.shape[0]
    m = 0.0
    for i in range(0, T, 4096):
        part = y_ref[i:i + 4096] - D[None, :, None].astype(np.float64) * x[i:i + 4096]
        m = max(m, float(np.max(np.abs(part), initial=0.0)))
    return m


SSM_REL_TOL = 1e-2   # bound on max|dy| / max|y_ref - D x| in bfloat16 mode
