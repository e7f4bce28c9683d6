"""The KDA oracle against its pins, and every planted mistake caught by at
least one pin (CPU only)."""
import pytest

from oracle import kda
from tests import kda_pins


@pytest.mark.parametrize("pin", kda_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_kda_pin(pin):
    assert kda.MUTATION == 0
    pin()


@pytest.mark.parametrize("m", sorted(kda._MUTATIONS), ids=lambda m: kda._MUTATIONS[m].replace(" ", "_"))
def test_kda_mutation_is_caught(m):
    kda.MUTATION = m
    try:
        failed = []
        for pin in kda_pins.ALL_PINS:
            try:
                pin()
            except AssertionError:
                failed.append(pin.__name__)
        assert failed, f"mutation {m} ({kda._MUTATIONS[m]}) passed every pin"
    finally:
        kda.MUTATION = 0
