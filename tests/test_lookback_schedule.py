"""Forward progress of the look-back prefill's ticket schedule (host logic; runs without a GPU).

The look-back launch hands out work through eight ticket counters, one per
residue of the workgroup index mod 8.  Counter x owns the whole sequences
[floor(x n / 8), floor((x+1) n / 8)) of the n = B * K_T sequences and hands out
their segments in segment-major order; the grid gives each residue
8 * ceil(n / 8) * nseg / 8 workgroups, and a workgroup whose ticket is past its
counter's items exits.  A segment waits for the segments before it in its own
sequence.  These tests restate that mapping (it is the one in
prefill_chunk_kernel.h) and check that

  * every predecessor of a segment is handed out earlier by the same counter,
    so a waiting workgroup only ever waits for a workgroup that started before
    it; and
  * a simulation of a GPU with a fixed number of workgroup slots, starting
    workgroups in several orders (in order, one XCD lagging behind the others,
    random), always drains the grid, including grids several times larger
    than the slots and sequence counts that are not a multiple of 8.
"""
import random

import pytest


def counter_items(nseq: int, nseg: int, x: int):
    lo, hi = (x * nseq) // 8, ((x + 1) * nseq) // 8
    nsx = hi - lo
    return [(lo + t % nsx, t // nsx) for t in range(nsx * nseg)] if nsx else []


def grid_size(nseq: int, nseg: int) -> int:
    return 8 * ((nseq + 7) // 8) * nseg


@pytest.mark.parametrize("nseq", [33, 39, 40, 41, 47, 63, 100, 129, 383])
@pytest.mark.parametrize("nseg", [1, 2, 7, 40])
def test_every_sequence_is_covered_once_and_predecessors_come_first(nseq, nseg):
    seen = {}
    for x in range(8):
        items = counter_items(nseq, nseg, x)
        assert len(items) <= grid_size(nseq, nseg) // 8
        for t, (s, g) in enumerate(items):
            assert (s, g) not in seen
            seen[(s, g)] = (x, t)
            if g > 0:
                px, pt = seen[(s, g - 1)]       # KeyError would mean "handed out later"
                assert px == x and pt < t
    assert len(seen) == nseq * nseg


def old_counter_items(nseq: int, nseg: int, x: int):
    """The replaced mapping: counter x hands out the global segment-major tickets x, x + 8, ..."""
    return [(t % nseq, t // nseq) for t in range(x, nseq * nseg, 8)]


def simulate(nseq: int, nseg: int, slots: int, order: str, seed: int = 0, mapping=counter_items,
             grid=None) -> int:
    """Start workgroups into `slots` slots in the given order; a started workgroup takes the next
    ticket of its counter, waits for its predecessor segment to finish, then runs one step.
    Returns the number of simulated steps; raises if the grid cannot drain."""
    rng = random.Random(seed)
    grid = grid_size(nseq, nseg) if grid is None else grid
    per_res = [list(range(x, grid, 8)) for x in range(8)]
    if order == "in_order":
        pending = list(range(grid))
    elif order == "lagging_xcd":          # residue 3 starts only when nothing else is left
        pending = [b for b in range(grid) if b % 8 != 3] + per_res[3]
    else:
        pending = list(range(grid))
        rng.shuffle(pending)
    items = [mapping(nseq, nseg, x) for x in range(8)]
    next_ticket = [0] * 8
    done = set()
    running = []                          # (sequence, segment) or None for padding
    steps = 0
    while pending or running:
        while pending and len(running) < slots:
            b = pending.pop(0)
            x = b % 8
            t = next_ticket[x]
            next_ticket[x] += 1
            running.append(items[x][t] if t < len(items[x]) else None)
        progressed = False
        still = []
        for it in running:
            if it is None or it[1] == 0 or (it[0], it[1] - 1) in done:
                if it is not None:
                    done.add(it)
                progressed = True
            else:
                still.append(it)
        running = still
        steps += 1
        if not progressed:
            raise AssertionError(f"deadlock: {len(running)} workgroups waiting, {len(pending)} not started")
    assert len(done) == nseq * nseg
    return steps


@pytest.mark.parametrize("order", ["in_order", "lagging_xcd", "random"])
@pytest.mark.parametrize("nseq,nseg,slots", [(39, 40, 1024), (39, 40, 64), (41, 25, 100),
                                              (47, 64, 1024), (100, 12, 256), (33, 8, 8)])
def test_grid_drains_under_any_start_order(order, nseq, nseg, slots):
    simulate(nseq, nseg, slots, order, seed=nseq * 31 + nseg)


def test_old_interleaved_mapping_can_deadlock_when_one_xcd_lags():
    """The mapping this replaces (counter x handing out the global tickets x, x+8, ... when the
    sequence count is not a multiple of 8) made segments wait on other counters' items: with one
    XCD's workgroups starting last and the slots full of waiters, the grid cannot drain.  The same
    start order drains with per-counter sequence ranges (test above)."""
    nseq, nseg = 39, 40
    simulate(nseq, nseg, 1024, "in_order", mapping=old_counter_items, grid=nseq * nseg)
    with pytest.raises(AssertionError, match="deadlock"):
        simulate(nseq, nseg, 64, "lagging_xcd", mapping=old_counter_items, grid=nseq * nseg)
