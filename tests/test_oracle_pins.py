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


def test_varlen_plan_partitions_sequences():
    """Packed-batch plan (oracle side): every sequence's items tile its tokens
    in order, none longer than the segment length; the items follow the
    longest-first order; the composite segments are each split sequence's
    segments but its last, and their sub-segments tile them in whole chunks."""
    # hand-worked: lengths 5, 1200, 0, 1200, 512 with 512-token segments
    cu = [0, 5, 1205, 1205, 2405, 2917]
    items, comps = oracle.varlen_plan(cu, 512, 2)
    assert items == [(1, 0, 5, 517), (1, 1, 517, 1029), (1, 2, 1029, 1205),
                     (3, 0, 1205, 1717), (3, 1, 1717, 2229), (3, 2, 2229, 2405),
                     (4, 0, 2405, 2917), (0, 0, 0, 5), (2, 0, 1205, 1205)]
    assert [(s, g) for s, g, _ in comps] == [(1, 0), (1, 1), (3, 0), (3, 1)]
    assert comps[0][2] == [(5, 261), (261, 517)]
    rng = np.random.default_rng(5)
    for trial in range(50):
        N = int(rng.integers(1, 20))
        lens = rng.integers(0, 3000, N)
        cu = np.concatenate([[0], np.cumsum(lens)])
        seg = int(rng.choice([0, 256, 512, 1024]))
        R = int(rng.integers(1, 9)) if seg == 0 else int(rng.integers(1, seg // 64 + 1))
        items, comps = oracle.varlen_plan(cu, seg, R)
        assert [s for s, g, *_ in items if g == 0] == sorted(range(N), key=lambda s: (-lens[s], s))
        for s in range(N):
            mine = [(g, a, b) for t, g, a, b in items if t == s]
            assert [g for g, _, _ in mine] == list(range(len(mine)))
            assert mine[0][1] == cu[s] and mine[-1][2] == cu[s + 1]
            assert all(x[2] == y[1] for x, y in zip(mine, mine[1:]))
            assert all(b - a <= seg for _, a, b in mine) or len(mine) == 1
            assert (len(mine) > 1) == (seg > 0 and lens[s] > seg)
            cs = [(g, subs) for t, g, subs in comps if t == s]
            assert [g for g, _ in cs] == list(range(len(mine) - 1))
            for g, subs in cs:
                assert subs[0][0] == mine[g][1] and subs[-1][1] == mine[g][2]
                assert all(x[1] == y[0] for x, y in zip(subs, subs[1:]))
                assert all((a - cu[s]) % 16 == 0 for a, _ in subs)
