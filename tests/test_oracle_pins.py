"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle
import oracle_pins


class _Orc:
    prefill = staticmethod(oracle.prefill)
    step = staticmethod(oracle.step)


@pytest.mark.parametrize("name", sorted(oracle_pins.PINS))
def test_pin(name):
    ok, detail = oracle_pins.PINS[name](_Orc)
    assert ok, f"pin {name} failed: {detail}"


class _LayerOrc:
    conv1d_step = staticmethod(oracle.conv1d_step)
    gated_rmsnorm = staticmethod(oracle.gated_rmsnorm)


@pytest.mark.parametrize("name", sorted(oracle_pins.LAYER_PINS))
def test_layer_pin(name):
    ok, detail = oracle_pins.LAYER_PINS[name](_LayerOrc)
    assert ok, f"pin {name} failed: {detail}"


class _S6Orc:
    selective_scan = staticmethod(oracle.selective_scan)
    prefill = staticmethod(oracle.prefill)


@pytest.mark.parametrize("name", sorted(oracle_pins.S6_PINS))
def test_selective_scan_pin(name):
    ok, detail = oracle_pins.S6_PINS[name](_S6Orc)
    assert ok, f"pin {name} failed: {detail}"


class _BwdOrc:
    prefill = staticmethod(oracle.prefill)
    prefill_backward = staticmethod(oracle.prefill_backward)


@pytest.mark.parametrize("name", sorted(oracle_pins.BWD_PINS))
def test_backward_pin(name):
    ok, detail = oracle_pins.BWD_PINS[name](_BwdOrc)
    assert ok, f"pin {name} failed: {detail}"


class _GdnOrc:
    gated_delta_rule = staticmethod(oracle.gated_delta_rule)


@pytest.mark.parametrize("name", sorted(oracle_pins.GDN_PINS))
def test_gated_delta_rule_pin(name):
    ok, detail = oracle_pins.GDN_PINS[name](_GdnOrc)
    assert ok, f"pin {name} failed: {detail}"
