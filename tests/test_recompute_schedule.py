"""The reverse pass's recompute schedules (diag_bwd_kernels.h): the tables compiled
into the kernel are the ones the generator prints, and simulating them on
symbolic states shows every reverse step gets the state after its token, in
order, with no more register slots than the kernel holds."""
import importlib.util
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bayesian_memory_scan_amd", "csrc")


def _generator():
    spec = importlib.util.spec_from_file_location("recompute_schedule",
                                                  os.path.join(CSRC, "recompute_schedule.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _tables():
    src = open(os.path.join(CSRC, "diag_bwd_kernels.h")).read()
    out = {}
    for m in re.finditer(r"struct RecSchedule<(\d+)> \{\s*static constexpr int N = (\d+);\s*"
                         r"static constexpr RecOp ops\[N\] = \{(.*?)\};\s*\};", src, re.S):
        rows = [tuple(int(x) for x in r.split(","))
                for r in re.findall(r"\{(-?\d+, -?\d+, -?\d+, -?\d+)\}", m.group(3))]
        assert len(rows) == int(m.group(2))
        out[int(m.group(1))] = rows
    return out


def simulate(rows, n, slots):
    """Run a schedule on symbolic states: a slot holds 'the state after token
    p' (p = -1: the checkpoint).  Returns (steps, copies)."""
    held = [None] * slots
    next_rev = n - 1
    steps = copies = 0
    for kind, src, dst, tok in rows:
        assert 0 <= src < slots and 0 <= dst < slots
        if kind == 0:
            held[dst] = -1
        elif kind == 1:
            assert held[src] == tok - 1, f"step {tok} reads the state after {held[src]}"
            if src != dst:
                copies += 1
            held[dst] = tok
            steps += 1
        else:
            assert kind == 2
            assert tok == next_rev, f"reverse of {tok}, expected {next_rev}"
            assert held[src] == tok, f"reverse of {tok} sees the state after {held[src]}"
            next_rev -= 1
    assert next_rev == -1, "not every token was reversed"
    return steps, copies


def test_tables_match_generator():
    gen = _generator()
    tables = _tables()
    assert set(tables) == {3, 4}
    for s in (3, 4):
        _, ops = gen.search(16, s)
        assert gen.assign(16, s, ops) == tables[s], f"{s}-slot table differs from the generator"


@pytest.mark.parametrize("slots,steps", [(3, 36), (4, 30)])
def test_tables_are_valid_and_short(slots, steps):
    got_steps, _ = simulate(_tables()[slots], 16, slots)
    assert got_steps == steps
    # holding `slots` consecutive states, each group rebuilt from the checkpoint
    grouped = sum(slots * m + min(slots, 16 - slots * m) for m in range((16 + slots - 1) // slots))
    assert got_steps < grouped


def test_simulator_rejects_a_wrong_table():
    rows = list(_tables()[3])
    kind, src, dst, tok = rows[1]
    rows[1] = (kind, src, dst, tok + 1)   # skip a token
    with pytest.raises(AssertionError):
        simulate(rows, 16, 3)
