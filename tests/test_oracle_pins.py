"""The oracle against its pins (CPU only)."""
import pytest

import oracle_pins

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


@pytest.mark.parametrize("name", sorted(oracle_pins.PINS))
def test_pin(name):
    oracle_pins.PINS[name]()
