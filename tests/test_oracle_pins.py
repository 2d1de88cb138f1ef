"""The oracle against its pins (CPU only)."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("name,fn,args", ALL_PINS, ids=[p[0] for p in ALL_PINS])
def test_pin(name, fn, args):
    fn(*args)
