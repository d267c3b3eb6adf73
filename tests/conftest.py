import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_terminal_summary(terminalreporter):
    """Print the error figures the GPU tests logged (max-abs errors against the
    oracle, per test and kernel variant), so a quiet run still shows them."""
    gpu_util = sys.modules.get("gpu_util")
    rec = getattr(gpu_util, "RECORD", None)
    if rec:
        terminalreporter.section("parity: errors against the fp64 oracle")
        for line in rec:
            terminalreporter.write_line(line)
