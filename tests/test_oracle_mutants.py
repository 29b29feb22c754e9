"""Negative controls: every planted mistake in the oracle must fail at least one pin.

Each mutant is the oracle built with -DORACLE_MUTANT=<n>, which changes one step
(swapped p/q in the accept test, resampling from p instead of the residual, strict top-p
inequality, highest-index ties, no renormalisation after top-k, accept length without
the extra token, wrong alpha, wrong Gumbel sign, temperature multiplying, top-k off by
one, Philox one round short, bonus at the wrong position, residual without the clamp, raw logprobs
in base 2, raw logprobs with the temperature applied, commit of the state after the drawn token's
position, commit with layers and rows swapped, sequence length grown by the accepted drafts only,
commit ignoring the slot map, slot commit one position late, slot commit that drops the old slot, tree draws that keep the rejected children, tree
children tested against their own mass alone, the parent's distribution after an accepted child, the
tree's final draw one depth late; the margin diagnostics: the accept distance taken over tests past the first
rejection, the Gumbel gap of the exponentiated keys, the top-p distance without the next larger value, and an
alternative draw that ignores the runner-up).
"""
import pytest

import oracle
import oracle_pins

MUTANTS = list(range(1, 30))


@pytest.mark.parametrize("mutant", MUTANTS)
def test_mutant_is_caught(mutant):
    o = oracle.Oracle(mutant=mutant, rebuild=True)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {mutant} passed every pin"
