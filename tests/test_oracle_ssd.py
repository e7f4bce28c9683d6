"""The SSD oracle against its pins, and every planted mistake caught by at
least one pin (CPU only)."""
import pytest

from oracle import ssd
from tests import ssd_pins


@pytest.mark.parametrize("pin", ssd_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_ssd_pin(pin):
    assert ssd.MUTATION == 0
    pin()


@pytest.mark.parametrize("m", sorted(ssd._MUTATIONS), ids=lambda m: ssd._MUTATIONS[m].replace(" ", "_"))
def test_ssd_mutation_is_caught(m):
    ssd.MUTATION = m
    try:
        failed = []
        for pin in ssd_pins.ALL_PINS:
            try:
                pin()
            except AssertionError:
                failed.append(pin.__name__)
        assert failed, f"mutation {m} ({ssd._MUTATIONS[m]}) passed every pin"
    finally:
        ssd.MUTATION = 0
