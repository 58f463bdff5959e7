"""The float64 oracle against the pages' worked examples, closed forms, invariants and the
pairwise brute-force definition (CPU only)."""
import pytest

from oracle_pins import ALL_PINS, Orc


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin, golden):
    pin(Orc(), golden)
