"""The CPU oracle checked against values it did not produce (library routines,
closed forms, the page's stated rules and printed example, invariants)."""
import os

import pytest

from oracle import oracle
from tests import oracle_pins_lib as pins

HERE = os.path.dirname(os.path.abspath(__file__))
CASES = pins.all_pins(oracle.run, oracle.round_half)


@pytest.mark.parametrize("name,check", CASES, ids=[c[0] for c in CASES])
def test_oracle_pin(name, check):
    check()


def test_projection_printed_example():
    pins.pin_gemm_example(oracle.projection, os.path.join(HERE, "golden", "gemm_worked_example.txt"))


def test_activation_entry_matches_library():
    import numpy as np
    xs = [-2.5, -0.7, -0.01, 0.0, 0.3, 0.45, 1.9]
    for name, (a, b) in pins.ACT_PARAMS.items():
        want = pins.library_activation(name, a, b, np.array(xs))
        got = [oracle.activation(name, a, b, x) for x in xs]
        pins.close(got, want, 1e-15, name)
