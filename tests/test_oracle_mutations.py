"""Plant each of a list of plausible mistakes in the oracle and check that some pin catches it.

The mistakes (selected in oracle.c by a switch that is off everywhere else): rotation sign flipped,
rotation pairs shifted by one dim, RMS over half the dims, gamma dropped, ReLU dropped, q read as
[128][64], head weights shifted by one head, ties broken toward the higher index, e4m3 ties away
from zero, the FNUZ maximum 240 instead of 448, bf16 truncation, visibility off by one, fp8 scale
dropped on dequantisation, a Hadamard butterfly stage skipped, the butterfly difference negated,
the Hadamard scale 1/128 instead of 2^-3.5, q quantised without dividing by its scale, the q
scale dropped from the fp8 x fp8 logit, e2m1 ties away from zero, fp4 nibbles swapped, the
attention's softmax scale dropped, a -1 list entry read as key 0, the kv slot of the next key
taken, the log-sum-exp without its maximum, q read as [512][heads], the fp8 quotient taken as a
product with the fp32 reciprocal of the scale, eps added outside the square root.
"""
import pytest

from tests.oracle_pins import ALL_PINS

MUTATIONS = list(range(1, 28))


@pytest.mark.parametrize("m", MUTATIONS)
def test_mutation_is_caught(oracle_mod, m):
    failed = []
    oracle_mod.set_mutation(m)
    try:
        for pin in ALL_PINS:
            try:
                pin()
            except Exception:  # noqa: BLE001 -- any failure of a pin counts
                failed.append(pin.__name__)
    finally:
        oracle_mod.set_mutation(0)
    assert failed, f"planted mistake {m} passed every pin"


def test_no_mutation_passes_all(oracle_mod):
    oracle_mod.set_mutation(0)
    for pin in ALL_PINS:
        pin()
