"""Pins for oracle.plan: hand-worked schedules, an independent tile-by-tile
construction, and the invariants any balanced schedule of this form obeys."""
import itertools
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.plan import build_plan, parse_plan, plan_size_words

HERE = os.path.dirname(__file__)
PAGE = 64


def _golden():
    with open(os.path.join(HERE, "golden", "plan_hand_worked.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_hand_worked_schedules(case):
    words = build_plan(case["seq_lens"], case["num_kv_heads"], case["n_workers"], case.get("entry_cost_q", 0))
    assert words.tolist() == case["words"]


def quota_walk(lens, H, W):
    """Independent construction: walk the tiles one by one, filling each
    worker up to its quota floor((w+1)T/W) - floor(wT/W), and merge runs of
    the same (worker, unit) into entries.  Returns per-worker entry lists."""
    tiles = [(b * H + h, j) for b in range(len(lens)) for h in range(H)
             for j in range((lens[b] + PAGE - 1) // PAGE)]
    T = len(tiles)
    quota = [((w + 1) * T) // W - (w * T) // W for w in range(W)]
    per_worker = [[] for _ in range(W)]
    w = 0
    for (u, j) in tiles:
        while quota[w] == 0:
            w += 1
        quota[w] -= 1
        run = per_worker[w]
        if run and run[-1][0] == u and run[-1][2] == j:
            run[-1][2] = j + 1
        else:
            run.append([u, j, j + 1])
    return per_worker


def priced_walk(lens, H, W, c):
    """Independent construction of the priced partition: tile by tile, with
    the running cost a = A(j + 1) after tile j, the tile goes to the worker
    w whose cost window (floor(w C / W), floor((w + 1) C / W)] holds a.
    Also checks the closed form owner(j) = floor((a W - 1) / C).  Returns
    per-worker entry lists, or None when the price does not apply."""
    tiles = [(b * H + h, j) for b in range(len(lens)) for h in range(H)
             for j in range((lens[b] + PAGE - 1) // PAGE)]
    T = len(tiles)
    cost = [4 + (c if j == 0 else 0) for (_, j) in tiles]
    C = sum(cost)
    if c == 0 or W > T or C < (4 + c + 1) * W or C >= 2**31:
        return None
    per_worker = [[] for _ in range(W)]
    w, a = 0, 0
    for (u, j), cj in zip(tiles, cost):
        a += cj
        while a > ((w + 1) * C) // W:
            w += 1
        assert w == (a * W - 1) // C
        run = per_worker[w]
        if run and run[-1][0] == u and run[-1][2] == j:
            run[-1][2] = j + 1
        else:
            run.append([u, j, j + 1])
    return per_worker


def check_plan(lens, H, W, c=0):
    words = build_plan(lens, H, W, c)
    p = parse_plan(words)
    U = len(lens) * H
    n = [(lens[u // H] + PAGE - 1) // PAGE for u in range(U)]
    T = sum(n)
    assert p["version"] == 1 and p["tile"] == PAGE
    assert (p["batch"], p["num_kv_heads"], p["n_workers"], p["n_tiles"]) == (len(lens), H, W, T)
    assert p["n_words"] == len(words) <= plan_size_words(len(lens), H, W)
    ents = p["entries"]
    wp = p["worker_ptr"]
    assert wp[0] == 0 and wp[-1] == p["n_entries"] and np.all(np.diff(wp) >= 0)

    # same schedule as the independent walk (the priced one when the price applies)
    priced = priced_walk(lens, H, W, c) if c else None
    assert p["entry_cost_q"] == (c if priced is not None else 0)
    walk = priced if priced is not None else quota_walk(lens, H, W)
    for w in range(W):
        got = [list(map(int, e[:3])) for e in ents[wp[w]:wp[w + 1]]]
        assert got == walk[w], (w, got, walk[w])

    # coverage: every tile of every unit exactly once
    seen = {u: np.zeros(n[u], dtype=int) for u in range(U)}
    for u, t0, t1, _ in ents:
        assert 0 <= t0 < t1 <= n[u]
        seen[int(u)][t0:t1] += 1
    assert all(np.all(v == 1) for v in seen.values())

    loads = [int(sum(e[2] - e[1] for e in ents[wp[w]:wp[w + 1]])) for w in range(W)]
    assert sum(loads) == T
    if priced is None:
        # balance: every worker holds floor(T/W) or ceil(T/W) tiles
        assert set(loads) <= {T // W, -(-T // W)}
    else:
        # every worker holds tiles, and its cost (4 per tile, c per entry
        # that starts a unit) is within one priced tile of its share C / W
        starts = [sum(1 for e in ents[wp[w]:wp[w + 1]] if e[1] == 0) for w in range(W)]
        costs = [4 * t + c * k for t, k in zip(loads, starts)]
        C = sum(costs)
        assert min(loads) >= 1
        assert all(C // W - (4 + c) < x < -(-C // W) + (4 + c) for x in costs), (costs, C)
    assert p["n_entries"] <= (W + U - 1 if T else 0)

    # slots: -1 exactly for single-entry units; otherwise a bijection onto [0, n_partials)
    count = {}
    for u, *_ in ents:
        count[int(u)] = count.get(int(u), 0) + 1
    slots = [int(e[3]) for e in ents]
    for e, s in zip(ents, slots):
        assert (s == -1) == (count[int(e[0])] == 1)
    split = sorted(s for s in slots if s >= 0)
    assert split == list(range(p["n_partials"]))
    # slots of one unit are consecutive, in entry order, units in increasing order
    prev_u, prev_s = -1, -1
    for u in sorted(count):
        us = [s for e, s in zip(ents, slots) if int(e[0]) == u and s >= 0]
        if us:
            assert us == list(range(us[0], us[0] + len(us))) and us[0] == prev_s + 1
            prev_s = us[-1]
    # merge list: every unit with 0 or >= 2 entries, increasing u
    comb = [tuple(map(int, c)) for c in p["combine"]]
    expect = []
    for u in range(U):
        c = count.get(u, 0)
        if c != 1:
            first = min((s for e, s in zip(ents, slots) if int(e[0]) == u), default=0)
            expect.append((u, c, first if c else 0))
    assert comb == expect
    return p


def test_exhaustive_single_sequence():
    for L in range(0, 131):
        for H in (1, 2):
            for W in range(1, 10):
                check_plan([L], H, W)


def test_exhaustive_two_sequences():
    vals = [0, 1, 37, 63, 64, 65, 127, 128, 129, 130]
    for a, b in itertools.product(vals, vals):
        for H in (1, 2):
            for W in range(1, 10):
                check_plan([a, b], H, W)


@settings(max_examples=300, deadline=None)
@given(lens=st.lists(st.integers(0, 5000), min_size=1, max_size=40),
       H=st.integers(1, 8), W=st.integers(1, 700))
def test_random_batches(lens, H, W):
    check_plan(lens, H, W)


PRICES = (1, 2, 4, 8, 16)


def test_priced_exhaustive_small():
    vals = [0, 1, 64, 65, 128, 200, 640]
    for a, b in itertools.product(vals, vals):
        for H in (1, 2):
            for W in range(1, 9):
                for c in PRICES:
                    check_plan([a, b, 64], H, W, c)


@settings(max_examples=300, deadline=None)
@given(lens=st.lists(st.integers(0, 5000), min_size=1, max_size=40),
       H=st.integers(1, 8), W=st.integers(1, 400), c=st.sampled_from(PRICES))
def test_priced_random_batches(lens, H, W, c):
    check_plan(lens, H, W, c)


def test_priced_reduces_to_plain():
    # a zero price, and a price the rule declines, give the plain plan word for word
    for lens, H, W in (([131072] + [4096] * 31, 1, 252), ([37, 64, 130, 200], 2, 5), ([64] * 9, 1, 9)):
        plain = build_plan(lens, H, W)
        assert np.array_equal(build_plan(lens, H, W, 0), plain)
    assert np.array_equal(build_plan([64] * 9, 1, 9, 8), build_plan([64] * 9, 1, 9))   # C = 108 < 13 * 9


def test_priced_workload_sizes():
    # skewed batch at W = 256: the price moves cuts but never empties a worker
    p = check_plan([131072] + [4096] * 31, 1, 256, 8)
    assert p["entry_cost_q"] == 8
    # 64 equal sequences of 8 tiles at W = 64: every share is one unit, priced or not
    p = check_plan([512] * 64, 1, 64, 8)
    assert p["n_partials"] == 0 and p["n_entries"] == 64


def test_workload_sizes():
    p = check_plan([131072] + [4096] * 31, 1, 256)
    assert p["n_tiles"] == 4032
    p = check_plan([512] * 64, 1, 256)
    assert p["n_tiles"] == 512 and p["n_partials"] == 256   # 2 tiles per worker: 4 entries per unit
    p = check_plan([37, 64, 130, 200], 1, 256)
    assert p["n_tiles"] == 9


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        build_plan([1, 2], 1, 0)
    with pytest.raises(ValueError):
        build_plan([1, -2], 1, 4)
    with pytest.raises(ValueError):
        build_plan([1, 2], 1, 4, -1)
