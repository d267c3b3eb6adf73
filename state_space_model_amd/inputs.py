"""Seeded synthetic inputs for the SSD prefill scan and decode step.

This module is shared by the GPU path's tests/benchmark and by the oracle's
tests.  It holds none of the scan's arithmetic: it only draws random inputs
with the shapes and distributions of the workloads below and rounds the bf16
operands to bfloat16 (round to nearest even) so that both sides consume the
exact same values.  Arrays are float32 numpy; operands that travel as bf16
hold bf16-representable values.

Draw order (fixed, generator ``numpy.random.Generator(PCG64(seed))``):
  0. packed-varlen workload only: lengths ~ integers[lo, hi] (inclusive)
  1. dt0_h = exp(U[log 1e-3, log 1e-1]);  b_h = log(expm1(dt0_h))  (inverse softplus)
  2. A_h   = -exp(U[log 1, log 16])
  3. D_h   ~ U[0, 1]
  4. x     ~ N(0, 1)                      [T, H, P]
  5. u     ~ N(0, 0.5^2)                  [T, H];  dt = softplus(u + b_h) in fp64 -> fp32
  6. B     ~ N(0, 1) / sqrt(N)            [T, G, N]
  7. C     ~ N(0, 1) / sqrt(N)            [T, G, N]
  8. h0    ~ N(0, 0.1^2)                  [nseq, H, N, P]  (when the workload has one)
The shapes are those of Mamba-2 layers (130M, 2.7B) and of a Codestral-7B
decode layer, as profiled in the pages: Compiler-First State Space Duality ...
(Tables 1-3, checkpoints 130M..2.7B at prompt lengths 1024-8192) and Mamba-2
SSD fused layer via VGpuWarp ("Lane mapping": 128 heads x head_dim 64,
d_state 128; conv_dim 10240 = 8192 + 2*8*128, i.e. 8 B/C groups).
"""
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" | "decode"
    H: int
    P: int
    N: int
    G: int
    dtype: str                # "f32" | "bf16": dtype of x, B, C on the device
    batch: int = 1            # dense batch (prefill) or decode batch
    L: int = 0                # dense sequence length (prefill)
    chunk: int = 256
    h0: bool = False
    steps: int = 1            # decode steps
    varlen: tuple = ()        # (nseq, lo, hi) for a packed variable-length batch
    chunks: tuple = field(default=())   # chunk sizes swept (packed varlen workload)


WORKLOADS = {
    0: Workload("tiny-prefill-f32", "prefill", H=4, P=16, N=16, G=1, dtype="f32",
                batch=1, L=256, chunk=64),
    1: Workload("mamba2-130m-layer-prefill", "prefill", H=24, P=64, N=128, G=1,
                dtype="bf16", batch=1, L=4096, chunk=256),
    2: Workload("mamba2-2.7b-layer-prefill", "prefill", H=80, P=64, N=128, G=1,
                dtype="bf16", batch=4, L=8192, chunk=256, h0=True),
    3: Workload("codestral-7b-decode-step", "decode", H=128, P=64, N=128, G=8,
                dtype="f32", batch=64, steps=128, h0=True),
    4: Workload("long-context-varlen-prefill", "prefill", H=80, P=64, N=128, G=1,
                dtype="bf16", chunk=256, h0=True, varlen=(8, 1024, 32768),
                chunks=(64, 128, 256, 512)),
}


def round_bf16(a):
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32).reshape(a.shape)


def _softplus(v):
    return np.logaddexp(0.0, v)


def _head_params(rng, H):
    dt0 = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=H))
    dt_bias = np.log(np.expm1(dt0))
    A = -np.exp(rng.uniform(np.log(1.0), np.log(16.0), size=H))
    D = rng.uniform(0.0, 1.0, size=H)
    return dt_bias, A.astype(np.float32), D.astype(np.float32)


def _draw_tokens(rng, lead, H, P, N, G, dt_bias, bf16):
    x = rng.standard_normal(size=lead + (H, P), dtype=np.float64).astype(np.float32)
    u = rng.normal(0.0, 0.5, size=lead + (H,))
    dt = _softplus(u + dt_bias).astype(np.float32)
    B = (rng.standard_normal(size=lead + (G, N)) / np.sqrt(N)).astype(np.float32)
    C = (rng.standard_normal(size=lead + (G, N)) / np.sqrt(N)).astype(np.float32)
    if bf16:
        x, B, C = round_bf16(x), round_bf16(B), round_bf16(C)
    return x, dt, B, C


def prefill_inputs(H, P, N, G, lengths, seed, dtype="bf16", h0=False):
    """Packed prefill inputs for sequences of the given lengths.

    Returns dict with x [T,H,P], dt [T,H], A [H], B/C [T,G,N], D [H],
    h0 [nseq,H,N,P] or None, cu_seqlens int64 [nseq+1].
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = np.asarray(lengths, dtype=np.int64)
    return _prefill_from(rng, H, P, N, G, lengths, dtype, h0)


def _prefill_from(rng, H, P, N, G, lengths, dtype, h0):
    T = int(lengths.sum())
    dt_bias, A, D = _head_params(rng, H)
    x, dt, B, C = _draw_tokens(rng, (T,), H, P, N, G, dt_bias, dtype == "bf16")
    h0a = None
    if h0:
        h0a = rng.normal(0.0, 0.1, size=(len(lengths), H, N, P)).astype(np.float32)
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, h0=h0a, cu_seqlens=cu)


def workload_inputs(k, seed=None):
    """Inputs of workload k with seed 1000+k (or `seed`)."""
    w = WORKLOADS[k]
    rng = np.random.Generator(np.random.PCG64(1000 + k if seed is None else seed))
    if w.kind == "decode":
        dt_bias, A, D = _head_params(rng, w.H)
        x, dt, B, C = _draw_tokens(rng, (w.steps, w.batch), w.H, w.P, w.N, w.G, dt_bias,
                                   w.dtype == "bf16")
        h = rng.normal(0.0, 0.1, size=(w.batch, w.H, w.N, w.P)).astype(np.float32)
        return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, h=h)
    if w.varlen:
        nseq, lo, hi = w.varlen
        lengths = rng.integers(lo, hi, endpoint=True, size=nseq)
    else:
        lengths = np.full(w.batch, w.L, dtype=np.int64)
    return _prefill_from(rng, w.H, w.P, w.N, w.G, lengths, w.dtype, w.h0)


def round_f16(a):
    """Round float32 values to the nearest float16 (ties to even); returns float32."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).astype(np.float32)


# The Mamba-1 selective-scan workload timed by COREY (section 5.1, Tables 2
# and 17): batch 1, d_inner 1024, L 4096, d_state 16, float16 activations.
S6_W1 = dict(name="mamba1-w1-selective-scan", batch=1, L=4096, dim=1024, N=16, dtype="f16")


def selective_scan_inputs(batch, L, dim, N, seed, dtype="f16", h0=False):
    """Seeded Mamba-1 selective-scan inputs, drawn in this order: per channel
    dt bias (as the SSD workloads), A[d][n] = -exp(U[log 1, log 16]),
    D ~ U[0,1]; per token x ~ N(0,1), dt = softplus(N(0,0.5^2) + bias),
    B, C ~ N(0,1)/sqrt(N); then h0 ~ N(0,0.1^2) if asked.  x, dt, B, C are
    rounded once to the operand dtype ("f32", "bf16" or "f16")."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dt0 = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=dim))
    bias = np.log(np.expm1(dt0))
    A = (-np.exp(rng.uniform(0.0, np.log(16.0), size=(dim, N)))).astype(np.float32)
    D = rng.uniform(0.0, 1.0, size=dim).astype(np.float32)
    x = rng.standard_normal(size=(batch, L, dim)).astype(np.float32)
    dt = _softplus(rng.normal(0.0, 0.5, size=(batch, L, dim)) + bias).astype(np.float32)
    B = (rng.standard_normal(size=(batch, L, N)) / np.sqrt(N)).astype(np.float32)
    C = (rng.standard_normal(size=(batch, L, N)) / np.sqrt(N)).astype(np.float32)
    h = rng.normal(0.0, 0.1, size=(batch, dim, N)).astype(np.float32) if h0 else None
    rnd = {"f32": lambda v: v, "bf16": round_bf16, "f16": round_f16}[dtype]
    return dict(x=rnd(x), dt=rnd(dt), A=A, B=rnd(B), C=rnd(C), D=D, h0=h)


def cotangents(T, nseq, H, P, N, seed, dtype="bf16", dh_out=True):
    """Seeded upstream gradients for the prefill's backward: dy [T,H,P] ~ N(0,1)
    (rounded to bfloat16 values for dtype "bf16", the type it is passed in) and
    dh_out [nseq,H,N,P] ~ N(0, 0.1^2) float32, or None."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dy = rng.standard_normal((T, H, P)).astype(np.float32)
    if dtype == "bf16":
        dy = round_bf16(dy)
    dh = rng.normal(0.0, 0.1, (nseq, H, N, P)).astype(np.float32) if dh_out else None
    return dy, dh


# Gated delta rule: a layer shape of the family Recurrence Scan names (its GDN
# layers), 32 value heads over 16 query/key groups, K = V = 128 (the pages give
# no shape; synthetic values stand in for a trained layer's activations).
GDN_W = dict(name="gdn-layer-prefill", batch=1, L=4096, H=32, G=16, K=128, V=128, dtype="bf16")


def gdn_inputs(lengths, H, G, K, V, seed, dtype="bf16", h0=False):
    """Seeded gated-delta-rule inputs for packed sequences: q ~ N(0,1)/sqrt(K),
    k = unit-norm N(0,1) rows, v ~ N(0,1) (q, k, v rounded to bf16 values for
    dtype "bf16" after normalising), gate g = log U[0.9, 1], beta = sigmoid of
    N(0,1), h0 ~ N(0, 0.1^2) when asked.  Returns a dict with cu_seqlens."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = np.asarray(lengths, dtype=np.int64)
    T = int(lengths.sum())
    q = (rng.standard_normal((T, G, K)) / np.sqrt(K)).astype(np.float32)
    k = rng.standard_normal((T, G, K))
    k = (k / np.maximum(np.linalg.norm(k, axis=-1, keepdims=True), 1e-6)).astype(np.float32)
    v = rng.standard_normal((T, H, V)).astype(np.float32)
    g = np.log(rng.uniform(0.9, 1.0, (T, H))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))).astype(np.float32)
    hz = rng.normal(0.0, 0.1, (len(lengths), H, V, K)).astype(np.float32) if h0 else None
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=hz, cu_seqlens=cu)
