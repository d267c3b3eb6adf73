"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that at least one pin catches each.  This is evidence that the pins constrain
every term of the recurrence, the state layout and the indexing."""
import functools
import os

import pytest

import oracle
from oracle import build as obuild
import oracle_pins

SRC = open(obuild.SRC).read()

_UPDATE = SRC[SRC.index("    for (int n = 0; n < N; ++n) {\n        const double bn"):SRC.index("    for (int p = 0; p < P; ++p) {\n        double acc")]
_OUTPUT = SRC[SRC.index("    for (int p = 0; p < P; ++p) {\n        double acc"):SRC.index("        y[p] = acc + D * (double)x[p];\n    }\n") + len("        y[p] = acc + D * (double)x[p];\n    }\n")]

# (name, exact original text, replacement)
MUTANTS = [
    ("decay-sign", "exp(dt * A)", "exp(-dt * A)"),
    ("decay-dropped", "a * h[(size_t)n * P + p] + dt", "h[(size_t)n * P + p] + dt"),
    ("decay-squared", "exp(dt * A)", "exp(2.0 * dt * A)"),
    ("dt-dropped-from-input", "dt * (double)x[p] * bn", "(double)x[p] * bn"),
    ("skip-dropped", "y[p] = acc + D * (double)x[p];", "y[p] = acc;"),
    ("skip-uses-dt", "y[p] = acc + D * (double)x[p];", "y[p] = acc + D * dt * (double)x[p];"),
    ("C-replaced-by-B", "acc += (double)C[n] * h", "acc += (double)B[n] * h"),
    ("output-before-update", _UPDATE + _OUTPUT, _OUTPUT + _UPDATE),
    ("group-modulo", "(int)(((long)hd * G) / H);", "(int)(hd % G);"),
    ("h0-ignored", "if (h0) memcpy(h, h0 + hoff", "if (0) memcpy(h, h0 + hoff"),
    ("last-token-dropped", "t < cu[s + 1]; ++t", "t + 1 < cu[s + 1]; ++t"),
    ("step-B-ignores-batch", "B + ((size_t)b * G + g) * N", "B + ((size_t)g) * N"),
    ("x-of-next-head", "x + ((size_t)t * H + hd) * P", "x + ((size_t)t * H + (hd + 1) % H) * P"),
]


@functools.lru_cache(maxsize=None)
def _mutant_lib(name, tmpdir):
    orig, repl = next((o, r) for n, o, r in MUTANTS if n == name)
    assert orig in SRC, f"mutation site for {name} not found in the oracle source"
    src = SRC.replace(orig, repl)
    path = os.path.join(tmpdir, f"mut_{name}.c")
    with open(path, "w") as f:
        f.write(src)
    lib = obuild.build(path, os.path.join(tmpdir, f"libmut_{name}.so"),
                       extra_flags=("-Wno-unused-variable", "-Wno-unused-but-set-variable"))
    return oracle.load(lib)


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_mutant_is_caught(name, tmp_path_factory):
    tmp = str(tmp_path_factory.getbasetemp())
    lib = _mutant_lib(name, tmp)

    class Orc:
        @staticmethod
        def prefill(*a, **k):
            return oracle.prefill(*a, lib=lib, **k)

        @staticmethod
        def step(*a, **k):
            return oracle.step(*a, lib=lib, **k)

    caught = []
    for pname, pin in oracle_pins.PINS.items():
        try:
            ok, _ = pin(Orc)
        except (ValueError, AssertionError, FloatingPointError):
            ok = False
        if not ok:
            caught.append(pname)
    assert caught, f"mutant {name} passed every pin"


# Planted mistakes in the decode-layer operations (conv1d step, gated norm);
# each must fail at least one of the layer pins.
LAYER_MUTANTS = [
    ("conv-newest-first", "wd[width - 1] = (double)u[(size_t)b * channels + c];",
     "wd[0] = (double)u[(size_t)b * channels + c];"),
    ("conv-no-shift", "wd[k] = wd[k + 1];", "wd[k] = wd[k];"),
    ("conv-bias-dropped", "double v = bias ? (double)bias[c] : 0.0;", "double v = 0.0;"),
    ("conv-tap-transposed", "v += (double)w[(size_t)c * width + k] * wd[k];",
     "v += (double)w[(size_t)c * width + (width - 1 - k)] * wd[k];"),
    ("conv-silu-sign", "v = v / (1.0 + exp(-v));", "v = v / (1.0 + exp(v));"),
    ("norm-sum-not-mean", "sqrt(ss / dim + eps)", "sqrt(ss + eps)"),
    ("norm-gate-dropped", "* (zz / (1.0 + exp(-zz)));", "* 1.0;"),
    ("norm-gate-sigmoid", "* (zz / (1.0 + exp(-zz)));", "* (1.0 / (1.0 + exp(-zz)));"),
    ("norm-weight-dropped", "*= r * (double)w[d];", "*= r;"),
    ("norm-eps-outside", "sqrt(ss / dim + eps)", "(sqrt(ss / dim) + eps)"),
]


@functools.lru_cache(maxsize=None)
def _layer_mutant_lib(name, tmpdir):
    orig, repl = next((o, r) for n, o, r in LAYER_MUTANTS if n == name)
    assert orig in SRC, f"mutation site for {name} not found in the oracle source"
    src = SRC.replace(orig, repl)
    path = os.path.join(tmpdir, f"lmut_{name}.c")
    with open(path, "w") as f:
        f.write(src)
    lib = obuild.build(path, os.path.join(tmpdir, f"liblmut_{name}.so"),
                       extra_flags=("-Wno-unused-variable", "-Wno-unused-but-set-variable"))
    return oracle.load(lib)


@pytest.mark.parametrize("name", [m[0] for m in LAYER_MUTANTS])
def test_layer_mutant_is_caught(name, tmp_path_factory):
    lib = _layer_mutant_lib(name, str(tmp_path_factory.getbasetemp()))

    class Orc:
        @staticmethod
        def conv1d_step(*a, **k):
            return oracle.conv1d_step(*a, lib=lib, **k)

        @staticmethod
        def gated_rmsnorm(*a, **k):
            return oracle.gated_rmsnorm(*a, lib=lib, **k)

    caught = []
    for pname, pin in oracle_pins.LAYER_PINS.items():
        try:
            ok, _ = pin(Orc)
        except (ValueError, AssertionError, FloatingPointError):
            ok = False
        if not ok:
            caught.append(pname)
    assert caught, f"mutant {name} passed every layer pin"



# Planted mistakes in the Mamba-1 selective scan; each must fail a selective-scan pin.
S6_MUTANTS = [
    ("s6-A-transposed", "exp(dtv * (double)A[(size_t)d * N + n])",
     "exp(dtv * (double)A[((size_t)n * dim + d) % ((size_t)dim * N)])"),
    ("s6-dt-of-channel-0", "const double dtv = (double)dt[td], xv",
     "const double dtv = (double)dt[td - d], xv"),
    ("s6-C-replaced-by-B", "acc += (double)Ct[n] * h[n];", "acc += (double)Bt[n] * h[n];"),
    ("s6-skip-dropped", "y[td] = acc + (double)D[d] * xv;", "y[td] = acc;"),
    ("s6-dt-dropped-from-input", "+ dtv * (double)Bt[n] * xv;", "+ (double)Bt[n] * xv;"),
    ("s6-h0-ignored", "h[n] = h0 ? h0[((size_t)b * dim + d) * N + n] : 0.0;", "h[n] = 0.0;"),
    ("s6-B-of-next-token", "const float *Bt = B + ((size_t)b * L + t) * N;",
     "const float *Bt = B + ((size_t)b * L + (t + 1) % L) * N;"),
]


@functools.lru_cache(maxsize=None)
def _s6_mutant_lib(name, tmpdir):
    orig, repl = next((o, r) for n, o, r in S6_MUTANTS if n == name)
    assert orig in SRC, f"mutation site for {name} not found in the oracle source"
    path = os.path.join(tmpdir, f"s6mut_{name}.c")
    with open(path, "w") as f:
        f.write(SRC.replace(orig, repl))
    lib = obuild.build(path, os.path.join(tmpdir, f"libs6mut_{name}.so"),
                       extra_flags=("-Wno-unused-variable", "-Wno-unused-but-set-variable"))
    return oracle.load(lib)


@pytest.mark.parametrize("name", [m[0] for m in S6_MUTANTS])
def test_selective_scan_mutant_is_caught(name, tmp_path_factory):
    lib = _s6_mutant_lib(name, str(tmp_path_factory.getbasetemp()))

    class Orc:
        @staticmethod
        def selective_scan(*a, **k):
            return oracle.selective_scan(*a, lib=lib, **k)

        @staticmethod
        def prefill(*a, **k):
            return oracle.prefill(*a, **k)   # the real SSD oracle: the reference side

    caught = []
    for pname, pin in oracle_pins.S6_PINS.items():
        try:
            ok, _ = pin(Orc)
        except (ValueError, AssertionError, FloatingPointError):
            ok = False
        if not ok:
            caught.append(pname)
    assert caught, f"mutant {name} passed every selective-scan pin"


# Planted mistakes in the reverse-mode gradients; each must fail a backward pin
# (the forward side of those pins is the real oracle).
BWD_MUTANTS = [
    ("bwd-skip-dropped-from-dx", "dxt[p] = Dh * dyt[p] + dtv * acc;", "dxt[p] = dtv * acc;"),
    ("bwd-ddt-decay-sign", "ddt[(size_t)t * H + hd] = Ah * a * da + gxb;",
     "ddt[(size_t)t * H + hd] = -Ah * a * da + gxb;"),
    ("bwd-adjoint-not-decayed", "= a_next * gg[(size_t)n * P + p] + (double)Ct[n]",
     "= gg[(size_t)n * P + p] + (double)Ct[n]"),
    ("bwd-dB-without-dt", "= dtv * bb;", "= bb;"),
    ("bwd-dA-without-dt", "dAacc += dtv * a * da;", "dAacc += a * da;"),
    ("bwd-dh0-not-decayed", "dh0[hoff + e] = a_next * gg[e];", "dh0[hoff + e] = gg[e];"),
    ("bwd-da-uses-new-state", "da += gv * hprev[(size_t)n * P + p];",
     "da += gv * ht[(size_t)n * P + p];"),
    ("bwd-dC-uses-old-state", "cb += ht[(size_t)n * P + p] * dyt[p];",
     "cb += hprev[(size_t)n * P + p] * dyt[p];"),
    ("bwd-dA-last-sequence-only", "sa += dAs[(size_t)s * H + hd];",
     "sa = dAs[(size_t)s * H + hd];"),
    ("bwd-dh_out-ignored", "if (dh_out) memcpy(gg, dh_out + hoff", "if (0) memcpy(gg, dh_out + hoff"),
    ("bwd-dD-without-x", "dDacc += dyt[p] * (double)xt[p];", "dDacc += dyt[p];"),
    ("bwd-group-sum-first-head", "if ((int)(((long)hd * G) / H) == g) {",
     "if (hd == g * (H / G)) {"),
]


@functools.lru_cache(maxsize=None)
def _bwd_mutant_lib(name, tmpdir):
    orig, repl = next((o, r) for n, o, r in BWD_MUTANTS if n == name)
    assert SRC.count(orig) == 1, f"mutation site for {name} not unique in the oracle source"
    path = os.path.join(tmpdir, f"bwdmut_{name}.c")
    with open(path, "w") as f:
        f.write(SRC.replace(orig, repl))
    lib = obuild.build(path, os.path.join(tmpdir, f"libbwdmut_{name}.so"),
                       extra_flags=("-Wno-unused-variable", "-Wno-unused-but-set-variable"))
    return oracle.load(lib)


@pytest.mark.parametrize("name", [m[0] for m in BWD_MUTANTS])
def test_backward_mutant_is_caught(name, tmp_path_factory):
    lib = _bwd_mutant_lib(name, str(tmp_path_factory.getbasetemp()))

    class Orc:
        @staticmethod
        def prefill(*a, **k):
            return oracle.prefill(*a, **k)   # the real forward oracle

        @staticmethod
        def prefill_backward(*a, **k):
            return oracle.prefill_backward(*a, lib=lib, **k)

    caught = []
    for pname, pin in oracle_pins.BWD_PINS.items():
        try:
            ok, _ = pin(Orc)
        except (ValueError, AssertionError, FloatingPointError):
            ok = False
        if not ok:
            caught.append(pname)
    assert caught, f"mutant {name} passed every backward pin"


# Planted mistakes in the gated delta rule; each must fail a delta-rule pin.
GDN_MUTANTS = [
    ("gdn-gate-missing-in-correction", "const double c = b * ((double)vt[i] - a * u[i]);",
     "const double c = b * ((double)vt[i] - u[i]);"),
    ("gdn-beta-dropped", "const double c = b * ((double)vt[i] - a * u[i]);",
     "const double c = ((double)vt[i] - a * u[i]);"),
    ("gdn-gate-sign", "const double a = exp((double)g[(size_t)t * H + hd]);",
     "const double a = exp(-(double)g[(size_t)t * H + hd]);"),
    ("gdn-output-reads-key", "acc += S[(size_t)i * K + j] * (double)qt[j];",
     "acc += S[(size_t)i * K + j] * (double)kt[j];"),
    ("gdn-correction-reads-query", "for (int j = 0; j < K; ++j) acc += S[(size_t)i * K + j] * (double)kt[j];\n                u[i] = acc;",
     "for (int j = 0; j < K; ++j) acc += S[(size_t)i * K + j] * (double)qt[j];\n                u[i] = acc;"),
    ("gdn-write-on-query", "S[(size_t)i * K + j] = a * S[(size_t)i * K + j] + c * (double)kt[j];",
     "S[(size_t)i * K + j] = a * S[(size_t)i * K + j] + c * (double)qt[j];"),
    ("gdn-h0-ignored", "if (h0) memcpy(S, h0 + soff", "if (0) memcpy(S, h0 + soff"),
    ("gdn-group-modulo", "const int gr = (int)(((long)hd * G) / H);", "const int gr = (int)(hd % G);"),
]


@functools.lru_cache(maxsize=None)
def _gdn_mutant_lib(name, tmpdir):
    orig, repl = next((o, r) for n, o, r in GDN_MUTANTS if n == name)
    assert SRC.count(orig) == 1, f"mutation site for {name} not unique in the oracle source"
    path = os.path.join(tmpdir, f"gdnmut_{name}.c")
    with open(path, "w") as f:
        f.write(SRC.replace(orig, repl))
    lib = obuild.build(path, os.path.join(tmpdir, f"libgdnmut_{name}.so"),
                       extra_flags=("-Wno-unused-variable", "-Wno-unused-but-set-variable"))
    return oracle.load(lib)


@pytest.mark.parametrize("name", [m[0] for m in GDN_MUTANTS])
def test_gated_delta_rule_mutant_is_caught(name, tmp_path_factory):
    lib = _gdn_mutant_lib(name, str(tmp_path_factory.getbasetemp()))

    class Orc:
        @staticmethod
        def gated_delta_rule(*a, **k):
            return oracle.gated_delta_rule(*a, lib=lib, **k)

    caught = []
    for pname, pin in oracle_pins.GDN_PINS.items():
        try:
            ok, _ = pin(Orc)
        except (ValueError, AssertionError, FloatingPointError):
            ok = False
        if not ok:
            caught.append(pname)
    assert caught, f"mutant {name} passed every delta-rule pin"
