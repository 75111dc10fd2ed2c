"""Pins for the static split-KV schedule of oracle.plan: hand-worked cases
under tests/golden/, and the properties its definition fixes (coverage,
share sizes, one entry per worker, slot bijection)."""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.plan import build_static_plan, parse_plan, static_split_count

HERE = os.path.dirname(__file__)
PAGE = 64


def _golden():
    with open(os.path.join(HERE, "golden", "static_plan_hand_worked.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_hand_worked_static_plans(case):
    p = parse_plan(build_static_plan(case["seq_lens"], case["num_kv_heads"], case["splits"]))
    assert p["n_workers"] == case["n_workers"]
    assert p["n_tiles"] == case["n_tiles"]
    assert p["n_partials"] == case["n_partials"]
    assert p["entries"].tolist() == case["entries"]
    assert p["combine"].tolist() == case["combine"]
    assert p["worker_ptr"].tolist() == [min(w, len(case["entries"])) for w in range(case["n_workers"] + 1)]


def check_static(lens, H, S):
    p = parse_plan(build_static_plan(lens, H, S))
    U = len(lens) * H
    n = [(lens[u // H] + PAGE - 1) // PAGE for u in range(U)]
    E = p["n_entries"]
    assert p["n_tiles"] == sum(n)
    assert p["n_workers"] == max(1, E)
    assert np.array_equal(p["worker_ptr"], np.minimum(np.arange(p["n_workers"] + 1), E))
    covered = [np.zeros(x, dtype=int) for x in n]
    per_unit = {}
    for u, t0, t1, slot in p["entries"].tolist():
        covered[u][t0:t1] += 1
        per_unit.setdefault(u, []).append((t0, t1, slot))
    assert all(np.all(c == 1) for c in covered)              # every tile exactly once
    slots = []
    for u in range(U):
        ents = per_unit.get(u, [])
        if n[u] == 0:
            assert not ents
            continue
        c = -(-n[u] // S)
        assert [e[0] for e in ents] == list(range(0, n[u], c))   # shares start at multiples of c_u
        assert all(t1 - t0 == c for t0, t1, _ in ents[:-1]) and 1 <= ents[-1][1] - ents[-1][0] <= c
        assert len(ents) <= S
        if len(ents) == 1:
            assert ents[0][2] == -1
        else:
            slots += [e[2] for e in ents]
    assert sorted(slots) == list(range(p["n_partials"]))      # slots are a bijection
    comb = {row[0]: (row[1], row[2]) for row in p["combine"].tolist()}
    for u in range(U):
        k = len(per_unit.get(u, []))
        assert (u in comb) == (k != 1)
        if k >= 2:
            assert comb[u] == (k, per_unit[u][0][2])
    return p


def test_single_split_is_one_worker_per_unit():
    p = check_static([37, 64, 130, 200, 0], 2, 1)
    assert p["n_workers"] == 8 and p["n_partials"] == 0


def test_skewed_batch_shares():
    lens = [131072] + [4096] * 31
    p = check_static(lens, 1, 8)
    sizes = p["entries"][:, 2] - p["entries"][:, 1]
    assert sizes[:8].tolist() == [256] * 8 and set(sizes[8:].tolist()) == {8}
    assert p["n_workers"] == 8 * 32


@settings(max_examples=300, deadline=None)
@given(lens=st.lists(st.integers(0, 20000), min_size=0, max_size=24), H=st.integers(1, 4),
       S=st.integers(1, 70))
def test_static_plan_properties(lens, H, S):
    check_static(lens, H, S)


def test_split_count_rule():
    assert static_split_count([131072] + [4096] * 31, 1, 256) == 8      # 32 units x 8 = 256
    assert static_split_count([512] * 64, 1, 256) == 4                  # 64 x 4 = 256
    assert static_split_count([1024] * 8, 1, 256) == 16                 # capped by 16 tiles
    assert static_split_count([100] * 300, 1, 256) == 1                 # already >= 256 units
    assert static_split_count([10 ** 6], 1, 256, max_splits=128) == 128
    assert static_split_count([0, 0], 1, 256) == 1


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        build_static_plan([10], 1, 0)
    with pytest.raises(ValueError):
        build_static_plan([-1], 1, 2)
