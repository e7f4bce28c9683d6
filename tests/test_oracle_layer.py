"""The oracle of the steps either side of the rule against its pins, and every
planted mistake caught by at least one pin (CPU only)."""
import pytest

from oracle import layer
from tests import layer_pins


@pytest.mark.parametrize("pin", layer_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_layer_pin(pin):
    assert layer.MUTATION == 0
    pin()


@pytest.mark.parametrize("m", sorted(layer._MUTATIONS), ids=lambda m: layer._MUTATIONS[m].replace(" ", "_"))
def test_layer_mutation_is_caught(m):
    layer.MUTATION = m
    try:
        failed = []
        for pin in layer_pins.ALL_PINS:
            try:
                pin()
            except AssertionError:
                failed.append(pin.__name__)
        assert failed, f"mutation {m} ({layer._MUTATIONS[m]}) passed every pin"
    finally:
        layer.MUTATION = 0
