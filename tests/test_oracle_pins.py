"""The CPU oracle against its pins (published vectors, printed values, library routines,
textbook samplers, closed forms and exact laws).  CPU only."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle(rebuild=True)


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(o, pin):
    pin(o)
