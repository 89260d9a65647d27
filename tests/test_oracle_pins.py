"""The CPU oracle against its pins (no GPU).  See tests/oracle_pins.py."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(0, force=False)


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(mutation=0)


# Each planted mistake (a dropped k term, B read with the wrong layout, ties
# rounded away from zero, truncation, a wrong bfloat16 exponent bias, a sign
# error; in the general form: beta ignored, a transposed A read as stored, B's
# leading dimension ignored; in the sampled entry points: a sample's row and
# column swapped, the old C's leading dimension ignored) must make at least
# one pin fail.
MUTATIONS = {
    1: "last k term dropped",
    2: "NN operand read as TN",
    3: "ties rounded away from zero",
    4: "truncation instead of rounding",
    5: "wrong bf16 exponent bias",
    6: "sign error on odd k",
    7: "general form ignores beta",
    8: "general form reads a transposed A as stored",
    9: "general form ignores the leading dimension of B",
    10: "general sampled form swaps a sample's row and column",
    11: "general sampled form ignores the leading dimension of the old C",
    12: "sampled TN/NN form swaps a sample's row and column",
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS), ids=lambda m: MUTATIONS[m])
def test_pins_catch_planted_mistake(mutation):
    oracle.build(mutation, force=False)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutation=mutation)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught planted mistake {mutation} ({MUTATIONS[mutation]})"
