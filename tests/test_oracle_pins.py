"""The float64 oracle against closed forms, invariants, torch library routines
and finite differences (see tests/oracle_pins.py for each pin's statement)."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    err, tol = pin()
    assert err <= tol, f"{pin.__name__}: error {err:.3e} > tolerance {tol:.1e}"
