"""The oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

from bwd_pins import BWD_PINS
from conv_pins import CONV_PINS
from epilogue_pins import DT_PINS, EPILOGUE_PINS, MERGE_PINS
from oracle import epilogue
from oracle import conv
from pins import ALL_PINS


@pytest.mark.parametrize("name", sorted(ALL_PINS))
def test_oracle_pin(name):
    fn, tol = ALL_PINS[name]
    err = fn(None)
    assert err <= tol, f"pin {name}: error {err} > {tol}"


@pytest.mark.parametrize("name", sorted(CONV_PINS))
def test_conv_oracle_pin(name):
    fn, tol = CONV_PINS[name]
    err = fn(conv)
    assert err <= tol, f"pin {name}: error {err} > {tol}"


@pytest.mark.parametrize("name", sorted(BWD_PINS))
def test_bwd_oracle_pin(name):
    fn, tol = BWD_PINS[name]
    err = fn(None)
    assert err <= tol, f"pin {name}: error {err} > {tol}"


@pytest.mark.parametrize("name", sorted(EPILOGUE_PINS))
def test_epilogue_oracle_pin(name):
    fn, tol = EPILOGUE_PINS[name]
    err = fn(epilogue)
    assert err <= tol, f"pin {name}: error {err} > {tol}"


@pytest.mark.parametrize("name", sorted(DT_PINS))
def test_dt_oracle_pin(name):
    from oracle import dt as odt
    fn, tol = DT_PINS[name]
    err = fn(odt)
    assert err <= tol, f"pin {name}: error {err} > {tol}"


@pytest.mark.parametrize("name", sorted(MERGE_PINS))
def test_merge_oracle_pin(name):
    from oracle import merge as omerge
    fn, tol = MERGE_PINS[name]
    err = fn(omerge)
    assert err <= tol, f"pin {name}: error {err} > {tol}"
