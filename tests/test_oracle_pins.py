"""The CPU oracle agrees with its pins (brute force, identities, invariants,
closed forms, library routines).  Runs on the CPU."""
import pytest

import pins


@pytest.mark.parametrize("name", list(pins.CHECKS))
def test_oracle_pin(name):
    fn, tol = pins.CHECKS[name]
    err = fn()
    assert err <= tol, f"{name}: error {err} > {tol}"
