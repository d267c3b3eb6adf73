"""MI355X-native Mamba-2 SSD selective scan (chunked prefill, decode step,
their gradients, and the related Mamba-1 and gated delta-rule scans).

The compute runs in the HIP library ``libssd.so`` (built from ``csrc/``);
``ssd.py`` is the thin ctypes binding over its C ABI (``include/ssd.h``).
Importing this package loads no library: the binding's entry points are
resolved on first attribute access, and the library on first call (which
raises if it has not been built).
"""

_API = ("prefill", "prefill_train", "prefill_backward", "step", "step_multi",
         "decode_layer_step", "selective_scan", "gated_delta_rule", "plan", "workspace_bytes")


def __getattr__(name):
    if name in _API:
        from . import ssd
        return getattr(ssd, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
