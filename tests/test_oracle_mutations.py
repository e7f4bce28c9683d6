"""Every planted mistake in the oracle must make at least one pin fail, so a
passing pin set is evidence rather than a no-op (CPU only)."""
import pytest

import oracle
from tests import pins

MUTATIONS = {
    1: "erase term dropped",
    2: "output read before the write",
    3: "decay applied after the erase read",
    4: "key not normalised",
    5: "1/sqrt(d_k) on k instead of q",
    6: "modulo key-head mapping",
    7: "softplus replaced by exp",
    8: "sign of g flipped",
    9: "beta = sigmoid(-b)",
    10: "output through the transposed state",
}


@pytest.mark.parametrize("m", sorted(MUTATIONS), ids=lambda m: MUTATIONS[m].replace(" ", "_"))
def test_mutation_is_caught(m):
    oracle.set_mutation(m)
    try:
        failed = []
        for pin in pins.ALL_PINS:
            try:
                pin()
            except AssertionError:
                failed.append(pin.__name__)
        assert failed, f"mutation {m} ({MUTATIONS[m]}) passed every pin"
    finally:
        oracle.set_mutation(0)
    assert oracle.get_mutation() == 0
