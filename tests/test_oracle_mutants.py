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
