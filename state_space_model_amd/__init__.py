"""MI355X-native Mamba-2 SSD selective scan (chunked prefill + decode step).

The compute runs in the HIP library ``libssd.so`` (built from ``csrc/``);
``ssd.py`` is the thin ctypes binding over its C ABI (``include/ssd.h``).
Importing this package does not load the library; ``prefill``/``step``/``step_multi``
load it on first use and raise if it is missing.
"""


def prefill(*args, **kwargs):
    from . import ssd
    return ssd.prefill(*args, **kwargs)


def step(*args, **kwargs):
    from . import ssd
    return ssd.step(*args, **kwargs)


def step_multi(*args, **kwargs):
    from . import ssd
    return ssd.step_multi(*args, **kwargs)


def decode_layer_step(*args, **kwargs):
    from . import ssd
    return ssd.decode_layer_step(*args, **kwargs)


def selective_scan(*args, **kwargs):
    from . import ssd
    return ssd.selective_scan(*args, **kwargs)


def prefill_backward(*args, **kwargs):
    from . import ssd
    return ssd.prefill_backward(*args, **kwargs)


def gated_delta_rule(*args, **kwargs):
    from . import ssd
    return ssd.gated_delta_rule(*args, **kwargs)


def prefill_train(*args, **kwargs):
    from . import ssd
    return ssd.prefill_train(*args, **kwargs)
