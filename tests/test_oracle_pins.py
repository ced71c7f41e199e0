"""The fp64 oracle against its pins (closed forms, library routines, invariants)."""
import pytest

from oracle import attention as oracle_impl
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle_impl)
