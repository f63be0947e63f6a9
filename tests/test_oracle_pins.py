"""The fp64 oracle against its pins (CPU only)."""
import pytest

from oracle_pins import ALL_PINS, backend


@pytest.fixture(scope="module")
def oracle_backend():
    import oracle
    oracle.load()
    return backend()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin, oracle_backend):
    pin(oracle_backend)
