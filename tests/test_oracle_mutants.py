"""Mutation check of the oracle pins.

Each mutant is the oracle with one planted slip (oracle.c, OR_MUTANT = k):
 1 fp16 scale rounded down instead of to nearest even
 2 nibble order swapped (low nibble = odd index)
 3 ties rounded away from zero instead of to even
 4 Hessian mean divides by M - 1
 5 residual grid s/16 instead of s/14
 6 Delta drops the e'^2 term
 7 Delta drops the Hessian weight
 8 ties in Delta broken by the higher block id
 9 residual partial sums land in the wrong group
10 output drops the residual term
11 dense partial sums pair x with the neighbouring weight
12 base error has the wrong sign
13 activation scale absmax/8 instead of absmax/7
14 migration factors with activation and weight ranges swapped
The mutants are built on the CPU into a temporary folder; the pins must fail
on every one of them.
"""
import inspect

import numpy as np
import pytest

import oracle
from tests import test_oracle_pins as pins

MUTANTS = list(range(1, 15))
PIN_FUNCS = [f for name, f in inspect.getmembers(pins, inspect.isfunction)
             if name.startswith("test_") and "orc" in inspect.signature(f).parameters]


@pytest.mark.parametrize("k", MUTANTS)
def test_pins_catch_planted_mistake(k, tmp_path):
    path = str(tmp_path / f"liboracle_mut{k}.so")
    oracle.build(extra_flags=[f"-DOR_MUTANT={k}"], out=path)
    orc = oracle.Oracle(path)
    caught = []
    for f in PIN_FUNCS:
        try:
            with np.errstate(all="ignore"):
                f(orc)
        except (AssertionError, ValueError) as exc:  # ValueError: oracle rejected its own output
            caught.append(f.__name__)
    assert caught, f"mutant {k} passed every pin"
