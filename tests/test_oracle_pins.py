"""The CPU oracle against closed forms, invariants, library routines, brute
force on tiny inputs and hand-worked fixtures (no GPU)."""
import pytest

import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check()
