"""Recompute schedules of the reverse pass (diag_bwd_kernels.h), printed as C++ tables.

The reverse pass walks a chunk's tokens last to first and needs, for token t,
the state after t.  Only the state before the chunk is stored (a
checkpoint); the others are rebuilt by forward steps into a few register
slots.  This script finds, for n tokens and s slots, the cheapest sequence of

  load  -> copy the checkpoint into a free slot
  step  -> advance a slot holding the state after t-1 by token t, in place or
           into a free slot (a copy costs the extra register moves)
  rev   -> run the reverse step of the next token (its state must be held)

by a shortest-path search over (tokens still to reverse, positions held),
then assigns concrete slot numbers.  Run:
  python3 recompute_schedule.py            # tables for 16 tokens, 3 and 4 slots
"""
import heapq
import sys

COPY_COST = 1.6    # a copy step: 32 fmacs + 32 moves against 32 fmacs in place
LOAD_COST = 0.05   # a checkpoint load: 8 vector loads, no VALU work


def search(n: int, s: int):
    start = (n, ())
    dist = {start: 0.0}
    prev = {}
    pq = [(0.0, start)]
    while pq:
        d, st = heapq.heappop(pq)
        if d > dist.get(st, float("inf")) + 1e-12:
            continue
        r, held = st
        if r == 0:
            ops = []
            while st in prev:
                st, op = prev[st]
                ops.append(op)
            return d, ops[::-1]

        def push(r2, h2, nd, op):
            ns = (r2, tuple(sorted(p for p in h2 if p <= r2 - 1)))
            if nd < dist.get(ns, float("inf")) - 1e-12:
                dist[ns] = nd
                prev[ns] = (st, op)
                heapq.heappush(pq, (nd, ns))

        if r - 1 in held:
            h = list(held)
            h.remove(r - 1)
            push(r - 1, h, d, ("rev", r - 1))
        if len(held) < s and -1 not in held:
            push(r, list(held) + [-1], d + LOAD_COST, ("load",))
        for p in set(held):
            if p + 1 > r - 1:
                continue
            h = list(held)
            h.remove(p)
            push(r, h + [p + 1], d + 1.0, ("step", p, True))
            if len(held) < s:
                push(r, list(held) + [p + 1], d + COPY_COST, ("step", p, False))
    raise RuntimeError("no schedule")


def assign(n: int, s: int, ops):
    """Slot numbers for the ops; returns (kind, src, dst, token) tuples."""
    slot = [None] * s          # position held by each slot
    out = []
    r = n
    for op in ops:
        if op[0] == "load":
            d = slot.index(None)
            slot[d] = -1
            out.append((0, d, d, -1))
        elif op[0] == "step":
            p, inplace = op[1], op[2]
            src = slot.index(p)
            dst = src if inplace else slot.index(None)
            slot[dst] = p + 1
            out.append((1, src, dst, p + 1))
        else:
            t = op[1]
            src = slot.index(t)
            out.append((2, src, src, t))
            r = t
            slot = [None if (x is None or x >= r) else x for x in slot]
    return out


def table(n: int, s: int) -> str:
    cost, ops = search(n, s)
    rows = assign(n, s, ops)
    body = ",\n".join("        {%d, %d, %d, %d}" % x for x in rows)
    return (f"// {n} tokens, {s} slots: {sum(1 for x in rows if x[0] == 1)} steps, "
            f"{sum(1 for x in rows if x[0] == 1 and x[1] != x[2])} of them copies, "
            f"{sum(1 for x in rows if x[0] == 0)} loads (cost {cost:.2f})\n"
            f"template <>\nstruct RecSchedule<{s}> {{\n"
            f"    static constexpr int N = {len(rows)};\n"
            f"    static constexpr RecOp ops[N] = {{\n{body}}};\n}};\n")


if __name__ == "__main__":
    n = int(sys.argv[1]) if len(sys.argv) > 1 else 16
    for s in (3, 4):
        print(table(n, s))
