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
# error) must make at least one pin fail.
MUTATIONS = {
    1: "last k term dropped",
    2: "NN operand read as TN",
    3: "ties rounded away from zero",
    4: "truncation instead of rounding",
    5: "wrong bf16 exponent bias",
    6: "sign error on odd k",
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
