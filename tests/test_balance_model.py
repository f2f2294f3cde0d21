"""A model of the prefill kernel's shared-tail protocol (Balance::take in
csrc/prefill.hip), run under random interleavings on the CPU.

The kernel itself can only run on the GPU; this test checks the protocol the
kernel implements, step by step as the hardware may order it: every tail
workgroup whose blockIdx is below `items` first adds 1 to the counter of the
XCD it runs on; a failed add, and every extra workgroup, reads the eight
counters one load at a time (other workgroups may act between the loads),
then adds to each queue whose loaded count was below the tail length, in
order from its own.  An add that returns i < tail takes item (stat + i) * 8 + y.
The invariants: every tail item is taken exactly once, every workgroup ends
after a bounded number of steps, and no static item is ever taken.  The XCD a
workgroup runs on is drawn at random (the protocol may not rely on
blockIdx % 8)."""

import random

import pytest

TAIL_PCT = 20  # Balance::kTailPct


def shares(items):
    per = items // 8
    stat = per - per * TAIL_PCT // 100
    return per, stat, per - stat


def take_steps(bid, x, items, stat, tail, counters):
    """Generator of one tail workgroup's atomic steps; yields after each
    memory operation and returns the item it takes, or -1."""
    if bid < items:
        i = counters[x]
        counters[x] += 1  # atomicAdd: the read and the add are one step
        yield
        if i < tail:
            return (stat + i) * 8 + x
    loaded = [0] * 8
    for y in range(8):  # eight relaxed loads, other workgroups interleave
        loaded[y] = counters[y]
        yield
    for k in range(8):
        y = (x + k) & 7
        if loaded[y] >= tail:
            continue
        i = counters[y]
        counters[y] += 1
        yield
        if i < tail:
            return (stat + i) * 8 + y
    return -1


def run_schedule(items, rng, xcd_of):
    per, stat, tail = shares(items)
    grid = items + items // 8
    counters = [0] * 8
    gens, taken = {}, {}
    for bid in range(8 * stat, grid):
        gens[bid] = take_steps(bid, xcd_of(bid), items, stat, tail, counters)
    steps = 0
    active = list(gens)
    while active:
        j = rng.randrange(len(active))
        bid = active[j]
        try:
            next(gens[bid])
            steps += 1
        except StopIteration as stop:
            taken[bid] = stop.value
            active[j] = active[-1]
            active.pop()
    return per, stat, tail, grid, taken, steps


@pytest.mark.parametrize("items", [768, 776, 1008, 1024, 4096, 8192])
def test_every_tail_item_taken_once(items):
    rng = random.Random(items)
    for trial in range(40 if items <= 1024 else 9):
        mode = trial % 3
        if mode == 0:
            xcd_of = lambda b: b % 8                  # round-robin placement
        elif mode == 1:
            xcd_of = lambda b: rng.randrange(8)       # any placement
        else:
            xcd_of = lambda b: 0                      # every tail workgroup on one XCD
        per, stat, tail, grid, taken, steps = run_schedule(items, rng, xcd_of)
        got = [t for t in taken.values() if t >= 0]
        want = sorted((stat + i) * 8 + y for y in range(8) for i in range(tail))
        assert sorted(got) == want, f"items {items} trial {trial}: tail items lost or taken twice"
        assert all(t < 0 or t >= 8 * stat for t in taken.values()), "a static item was handed out"
        n_tail_wg = grid - 8 * stat
        assert len(taken) == n_tail_wg                # every workgroup ended
        assert steps <= n_tail_wg * (1 + 8 + 8)       # at most one add, eight loads and eight adds each


def test_shares_match_the_launch():
    """The static part is a whole number of items per XCD, the tail is about
    20 % of each XCD's list, and the grid leaves at least one tail workgroup
    per tail item."""
    for items in range(768, 20000, 8):
        per, stat, tail = shares(items)
        assert stat + tail == per and tail >= 0
        assert abs(tail - per * TAIL_PCT / 100) < 1
        grid = items + items // 8
        assert grid - 8 * stat >= 8 * tail
