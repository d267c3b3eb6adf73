"""Helpers for the GPU parity tests: upload seeded inputs, sample heads for
the oracle, compare.  Inputs come from state_space_model_amd.inputs; expected
values come only from the oracle."""
import sys

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}   # max-abs on every compared element of y and h_out


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


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


def maxabs(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    return float(np.max(np.abs(a - b), initial=0.0))
