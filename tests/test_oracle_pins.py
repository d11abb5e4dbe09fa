"""The CPU oracle against what the pages and mathematics fix (runs on CPU)."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_plan_partitions_tokens():
    """P-11 (oracle side): chunks tile [0, T) in order with only the last one
    ragged, and segments are unions of whole chunks covering [0, T)."""
    for T in (1, 2, 15, 16, 17, 64, 2048, 16383, 16384, 65537):
        for C in (1, 8, 16, 32, 64):
            starts, lens, bounds = oracle.plan(T, C, 1)
            assert sum(lens) == T and starts[0] == 0
            assert all(s + l == n for s, l, n in zip(starts, lens, starts[1:]))
            assert all(l == C for l in lens[:-1]) and 1 <= lens[-1] <= C
            for S in (1, 2, 3, 4, 7, 64):
                _, _, b = oracle.plan(T, C, S)
                assert b[0] == 0 and b[-1] == T and len(b) == S + 1
                assert all(x <= y for x, y in zip(b, b[1:]))
                assert all(x % C == 0 for x in b[:-1])


def test_element_offset_beyond_int32():
    off = oracle.element_offset(255, 15, 16383, 127, H=16, T=16384, D=128)
    assert off == 256 * 16 * 16384 * 128 - 1 and off > 2**31
