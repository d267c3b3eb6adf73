"""The fp64 oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only), run over every entry point on small ragged inputs: empty and
one-token sequences, no initial state, odd sizes.  Any out-of-bounds access,
use of freed memory or undefined arithmetic aborts the child process; its
results must also equal those of the normal build."""
import os
import subprocess
import sys

import pytest

from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys
import numpy as np
sys.path.insert(0, sys.argv[2])
import oracle
from state_space_model_amd import inputs

san = oracle.load(sys.argv[1])
ref = oracle.load()

def same(a, b):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape and np.allclose(a, b, rtol=1e-12, atol=1e-12), "sanitized build differs"

for lengths, H, P, N, G, h0 in [([40, 0, 7, 1], 3, 16, 16, 1, True), ([5], 4, 7, 3, 2, False),
                                ([0], 2, 8, 4, 1, True), ([1, 1], 6, 3, 5, 3, True)]:
    d = inputs.prefill_inputs(H, P, N, G, lengths, 11, dtype="f32", h0=h0)
    h = None if d["h0"] is None else d["h0"].astype(np.float64)
    args = (d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"])
    for a, b in zip(oracle.prefill(*args, h, d["cu_seqlens"], lib=san),
                    oracle.prefill(*args, h, d["cu_seqlens"], lib=ref)):
        same(a, b)
    T = int(sum(lengths))
    dy, dh = inputs.cotangents(T, len(lengths), H, P, N, 12, "f32", dh_out=h0)
    g1 = oracle.prefill_backward(*args, dy, h, dh, d["cu_seqlens"], lib=san)
    g2 = oracle.prefill_backward(*args, dy, h, dh, d["cu_seqlens"], lib=ref)
    for k in g1:
        same(g1[k], g2[k])
    if T > 0:
        b = min(T, 3)
        st1 = np.random.default_rng(1).normal(size=(b, H, N, P))
        st2 = st1.copy()
        same(oracle.step(d["x"][:b], d["dt"][:b], d["A"], d["B"][:b], d["C"][:b], d["D"], st1, lib=san),
             oracle.step(d["x"][:b], d["dt"][:b], d["A"], d["B"][:b], d["C"][:b], d["D"], st2, lib=ref))
        same(st1, st2)

rng = np.random.default_rng(2)
u, w, bias = rng.normal(size=(3, 10)), rng.normal(size=(10, 4)), rng.normal(size=10)
w1, w2 = rng.normal(size=(3, 10, 4)), None
w2 = w1.copy()
same(oracle.conv1d_step(u, w1, w, bias, lib=san), oracle.conv1d_step(u, w2, w, bias, lib=ref))
same(w1, w2)
yv, z, nw = rng.normal(size=(2, 9)), rng.normal(size=(2, 9)), rng.normal(size=9)
same(oracle.gated_rmsnorm(yv, z, nw, lib=san), oracle.gated_rmsnorm(yv, z, nw, lib=ref))

s6 = inputs.selective_scan_inputs(2, 9, 5, 4, 13, dtype="f32", h0=True)
a6 = (s6["x"], s6["dt"], s6["A"], s6["B"], s6["C"], s6["D"], s6["h0"])
for a, b in zip(oracle.selective_scan(*a6, lib=san), oracle.selective_scan(*a6, lib=ref)):
    same(a, b)

dg = inputs.gdn_inputs([9, 0, 4], 4, 2, 8, 6, 14, dtype="f32", h0=True)
ag = (dg["q"], dg["k"], dg["v"], dg["g"], dg["beta"], dg["h0"].astype(np.float64), dg["cu_seqlens"])
for a, b in zip(oracle.gated_delta_rule(*ag, lib=san), oracle.gated_delta_rule(*ag, lib=ref)):
    same(a, b)
print("SANITIZED_OK")
'''


def _libasan():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    asan = _libasan()
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = oracle_build.build(out=str(tmp_path / "liboracle_san.so"),
                             extra_flags=("-fsanitize=address,undefined",
                                          "-fno-sanitize-recover=undefined",
                                          "-fno-omit-frame-pointer", "-g"))
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", CHILD, lib, ROOT], capture_output=True, text=True,
                       env=env, timeout=600)
    assert r.returncode == 0 and "SANITIZED_OK" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
