"""The worker-count rule (hpc_decode_choose_workers), host only.

Its definition, written out here: worker w of W holds global tiles
[floor(w T / W), floor((w + 1) T / W)) of the unit-major tile list; it costs
its tile count plus entry_cost for every unit with tiles that its range
touches; the rule scans W down from hi to lo and keeps a smaller W only when
its costliest worker prices at least 1% below the best so far.
"""
import ctypes

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import load_balanced_paged_step_amd as hd
from oracle.plan import build_plan, parse_plan, priced_boundaries
from workloads import WORKLOADS, workload_inputs, workload_lengths


MIN_GAIN = 0.01   # a smaller W must price at least 1% below the best larger one


def _brute(lens, H, lo, hi, ce):
    units = []
    start = 0
    for L in lens:
        n = -(-int(L) // 64)
        for _ in range(H):
            if n:
                units.append((start, start + n))
                start += n
    T = start
    if T == 0:
        return hi
    best, best_cost = None, None
    for W in range(hi, lo - 1, -1):
        worst = 0.0
        for w in range(W):
            a, b = w * T // W, (w + 1) * T // W
            if a == b:
                continue
            worst = max(worst, (b - a) + ce * sum(1 for s, e in units if s < b and e > a))
        if best is None or worst < best_cost * (1 - MIN_GAIN) - 1e-9:
            best, best_cost = W, worst
    return best


def test_skewed_batch_takes_the_aligned_worker_count():
    """1 x 128K + 31 x 4K, one KV head: T = 4032 = 16 x 252, so at W = 252
    every sequence boundary is a worker boundary and each worker holds one
    entry (16 tiles + 0.5), against 16 tiles and two entries for some of the
    256 workers."""
    lens = workload_lengths(4)
    assert hd.hpc_decode_choose_workers(lens, 1, 128, 256) == 252
    assert hd.hpc_decode_choose_workers(lens, 1, 253, 256) == 256      # 252 outside the window
    assert _brute(lens, 1, 240, 256, 0.5) == 252


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_batches_without_a_better_count_keep_every_worker(cfg):
    assert hd.hpc_decode_choose_workers(workload_lengths(cfg), WORKLOADS[cfg].num_kv_heads, 128, 256) == 256


def test_without_an_entry_price_the_largest_count_wins():
    """Tiles alone: the costliest worker holds ceil(T / W) tiles, which never
    grows with W, and ties go to the larger W."""
    rng = np.random.default_rng(3)
    for _ in range(20):
        lens = rng.integers(0, 5000, size=rng.integers(1, 12))
        assert hd.hpc_decode_choose_workers(lens, 2, 10, 90, 0.0) == 90


@settings(max_examples=60, deadline=None)
@given(lens=st.lists(st.integers(0, 3000), min_size=1, max_size=9), H=st.integers(1, 3),
       lo=st.integers(1, 40), span=st.integers(0, 40), ce=st.sampled_from([0.0, 0.25, 0.5, 1.0, 3.0]))
def test_matches_the_definition(lens, H, lo, span, ce):
    assert hd.hpc_decode_choose_workers(np.array(lens), H, lo, lo + span, ce) == _brute(lens, H, lo, lo + span, ce)


def test_errors():
    lib = hd.lib()
    lens = np.array([100, 200], dtype=np.int32)
    p = lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert lib.hpc_decode_choose_workers(p, 2, 1, 1, 8, 0.5) >= 1
    assert lib.hpc_decode_choose_workers(None, 2, 1, 1, 8, 0.5) == hd.HPC_ERR_NULL
    assert lib.hpc_decode_choose_workers(None, 0, 1, 1, 8, 0.5) == 8                    # empty batch
    assert lib.hpc_decode_choose_workers(p, -1, 1, 1, 8, 0.5) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_choose_workers(p, 2, 0, 1, 8, 0.5) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_choose_workers(p, 2, 1, 0, 8, 0.5) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_choose_workers(p, 2, 1, 9, 8, 0.5) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_choose_workers(p, 2, 1, 1, 8, -0.1) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_choose_workers(p, 2, 1, 1, 8, float("nan")) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_choose_workers(p, 2, 1, 1, 8, float("inf")) == hd.HPC_ERR_INVALID
    bad = np.array([100, -1], dtype=np.int32)
    assert lib.hpc_decode_choose_workers(bad.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 2, 1, 1, 8,
                                         0.5) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_choose_workers(np.zeros(3, np.int32).ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 3,
                                         2, 4, 8, 0.5) == 8                             # no tiles


@pytest.mark.parametrize("cfg,expected", [(1, 256), (2, 256), (3, 256), (4, 252), (5, 512)])
def test_pick_workers_on_the_decode_workloads(cfg, expected):
    """One worker per CU at the rule's count, except the fp8 batch (64q/8kv,
    2 entries per worker at W = 255): two per CU."""
    w = WORKLOADS[cfg]
    assert hd.hpc_decode_pick_workers(workload_lengths(cfg), w.num_kv_heads, w.kv_dtype, 256) == expected


def test_pick_workers_rule():
    lens5 = workload_lengths(5)
    # the same lengths on a bf16 cache: one per CU at the rule's count
    assert hd.hpc_decode_pick_workers(lens5, 8, "bf16", 256) == hd.hpc_decode_choose_workers(lens5, 8, 128, 256)
    # fp8 with one entry per worker (16 x 32K, 8 KV heads: 128 units of 512 tiles, half a unit per worker)
    assert hd.hpc_decode_pick_workers(np.full(16, 32768), 8, "fp8_e4m3", 256) == 256
    # fp8 with exactly two whole units per worker (64 x 4K, 8 KV heads) goes to two per CU
    assert hd.hpc_decode_pick_workers(np.full(64, 4096), 8, "fp8_e4m3", 256) == 512
    # the threshold is 1.5 entries per worker: 3 units over 2 workers -> 2 entries each when split in the middle
    assert hd.hpc_decode_pick_workers(np.full(3, 64 * 4), 1, "fp8_e4m3", 2) == 4
    assert hd.hpc_decode_pick_workers(np.full(2, 64 * 4), 1, "fp8_e4m3", 2) == 2
    assert hd.hpc_decode_pick_workers(np.zeros(4, np.int32), 1, "fp8_e4m3", 64) == 64      # no tiles


def test_pick_workers_errors():
    lib = hd.lib()
    lens = np.array([100, 200], dtype=np.int32)
    p = lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert lib.hpc_decode_pick_workers(p, 2, 1, hd.HPC_KV_BF16, 256) >= 1
    assert lib.hpc_decode_pick_workers(None, 2, 1, hd.HPC_KV_BF16, 256) == hd.HPC_ERR_NULL
    assert lib.hpc_decode_pick_workers(p, 2, 1, hd.HPC_KV_BF16, 1) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_pick_workers(p, 2, 1, 7, 256) == hd.HPC_ERR_UNSUPPORTED
    assert lib.hpc_decode_pick_workers(p, -1, 1, hd.HPC_KV_BF16, 256) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_pick_workers(p, 2, 0, hd.HPC_KV_FP8_E4M3, 256) == hd.HPC_ERR_INVALID


@pytest.mark.parametrize("cfg", [1, 4, 5])
def test_workload_lengths_match_the_inputs(cfg):
    assert np.array_equal(workload_lengths(cfg), workload_inputs(cfg).seq_lens.numpy())


def test_near_ties_keep_the_larger_count():
    """The fp8 batch's lengths price 207.0 tiles at 255 workers against 207.5
    at 256 (0.24% cheaper): not enough to leave a compute unit idle."""
    lens5 = workload_lengths(5)
    assert hd.hpc_decode_choose_workers(lens5, 8, 128, 256) == 256
    assert _brute(lens5, 8, 250, 256, 0.5) == 256


def test_trace_window_errors():
    """The tracing window's host calls check their arguments and call no HIP."""
    lib = hd.lib()
    assert lib.hpc_decode_trace_start(None, 4096) == hd.HPC_ERR_NULL
    assert lib.hpc_decode_trace_start(ctypes.c_void_p(0x1000), 63) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_trace_start(ctypes.c_void_p(0x1000), 64) == hd.HPC_OK
    assert lib.hpc_decode_trace_stop() == hd.HPC_OK


# ------------------------------------------------ entry price of the partition ---

ENTRY_COST = {"bf16": 0.5, "fp8_e4m3": 2.0}


def _brute_price(lens, H, W, kv):
    """The price rule written out: each candidate price's partition (the
    oracle's priced boundaries) costs its costliest worker's tiles plus
    ENTRY_COST per unit its range touches; scanning 0, 2, 4, 8, 16, a price
    replaces the best only when 1% cheaper, and a declined price is skipped."""
    n = [-(-int(L) // 64) for L in lens for _ in range(H)]
    units, start = [], 0
    for k in n:
        if k:
            units.append((start, start + k))
        start += k
    if start == 0:
        return 0
    ce = ENTRY_COST[kv]
    best, best_cost = None, None
    for c in (0, 2, 4, 8, 16):
        s, applied = priced_boundaries(n, W, c)
        if c and not applied:
            continue
        worst = 0.0
        for w in range(W):
            a, b = s[w], s[w + 1]
            if a < b:
                worst = max(worst, (b - a) + ce * sum(1 for u0, u1 in units if u0 < b and u1 > a))
        if best is None or worst < best_cost * (1 - MIN_GAIN) - 1e-9:
            best, best_cost = c, worst
    return best


@pytest.mark.parametrize("cfg,W,expected", [(4, 252, 0), (4, 256, 4), (5, 512, 8), (5, 256, 8)])
def test_pick_entry_price_on_the_decode_workloads(cfg, W, expected):
    """The skewed batch at 252 workers fits unit boundaries exactly (price 0);
    at 256 a small price removes second entries; the fp8 batch, with about
    two entries per worker, takes 8 quarter tiles at either worker count."""
    w = WORKLOADS[cfg]
    lens = workload_lengths(cfg)
    got = hd.hpc_decode_pick_entry_price(lens, w.num_kv_heads, w.kv_dtype, W)
    assert got == expected == _brute_price(lens, w.num_kv_heads, W, w.kv_dtype)


@settings(max_examples=80, deadline=None)
@given(lens=st.lists(st.integers(0, 6000), min_size=1, max_size=12), H=st.integers(1, 4),
       W=st.integers(1, 60), kv=st.sampled_from(["bf16", "fp8_e4m3"]))
def test_pick_entry_price_matches_the_definition(lens, H, W, kv):
    assert hd.hpc_decode_pick_entry_price(np.array(lens), H, kv, W) == _brute_price(lens, H, W, kv)


def test_pick_entry_price_errors():
    lib = hd.lib()
    lens = np.array([100, 200], dtype=np.int32)
    p = lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert lib.hpc_decode_pick_entry_price(p, 2, 1, hd.HPC_KV_BF16, 4) >= 0
    assert lib.hpc_decode_pick_entry_price(None, 2, 1, hd.HPC_KV_BF16, 4) == hd.HPC_ERR_NULL
    assert lib.hpc_decode_pick_entry_price(None, 0, 1, hd.HPC_KV_BF16, 4) == 0           # empty batch
    assert lib.hpc_decode_pick_entry_price(p, -1, 1, hd.HPC_KV_BF16, 4) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_pick_entry_price(p, 2, 0, hd.HPC_KV_BF16, 4) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_pick_entry_price(p, 2, 1, hd.HPC_KV_BF16, 0) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_pick_entry_price(p, 2, 1, 7, 4) == hd.HPC_ERR_UNSUPPORTED
    bad = np.array([100, -1], dtype=np.int32)
    assert lib.hpc_decode_pick_entry_price(bad.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 2, 1,
                                           hd.HPC_KV_BF16, 4) == hd.HPC_ERR_INVALID


# ------------------------------------------------------ merge mode of the step ---

def _oracle_max_shares(lens, H, W, price):
    """Most workers sharing one unit, read off the oracle plan's merge records
    (each record holds a split unit's worker count), and the plan's tile count."""
    plan = parse_plan(build_plan(np.asarray(lens, dtype=np.int64), H, W, entry_cost_q=price))
    return max([1] + [int(r[1]) for r in plan["combine"]]), plan["n_tiles"]


def _rule(lens, H, W, price):
    """The merge rule written out: in the kernel when nothing is split, or
    when there are no more tiles than workers and no unit has more than
    FUSED_MAX_SHARES workers."""
    most, T = _oracle_max_shares(lens, H, W, price)
    return most == 1 or (T <= W and most <= hd.FUSED_MAX_SHARES)


@pytest.mark.parametrize("lens,H,W,expected", [
    ([37, 80, 150, 200], 1, 256, True),          # 10 tiles, up to 4 workers a unit
    ([512] * 8, 1, 256, True),                   # 64 tiles, 8 workers a unit
    ([1024] * 8, 1, 256, False),                 # 128 tiles, 16 workers a unit
    ([512] * 64, 1, 256, False),                 # more tiles than workers
    ([131072] + [4096] * 31, 1, 252, False),     # the long sequence over 128 workers
    ([4096] * 64, 1, 64, True),                  # no unit split: no merge kernel to launch
    ([0, 0, 0], 2, 16, True),                    # no tiles at all
])
def test_pick_merge_cases(lens, H, W, expected):
    assert hd.hpc_decode_pick_merge(np.array(lens), H, W) is expected
    assert _rule(lens, H, W, 0) is expected


def test_pick_merge_on_the_decode_workloads():
    """At the rules' worker count and price: the in-kernel merge for the tiny
    batch only (10 tiles); the uniform batch has more tiles than workers, and
    8 x 1K, the 128K sequence and the fp8 batch's long sequences spread over
    more than 8 workers."""
    got = {}
    for cfg, w in WORKLOADS.items():
        lens = workload_lengths(cfg)
        W = hd.hpc_decode_pick_workers(lens, w.num_kv_heads, w.kv_dtype, 256)
        price = hd.hpc_decode_pick_entry_price(lens, w.num_kv_heads, w.kv_dtype, W)
        got[cfg] = hd.hpc_decode_pick_merge(lens, w.num_kv_heads, W, price)
        assert got[cfg] is _rule(lens, w.num_kv_heads, W, price)
    assert got == {1: True, 2: False, 3: False, 4: False, 5: False}


@settings(max_examples=80, deadline=None)
@given(lens=st.lists(st.integers(0, 6000), min_size=1, max_size=12), H=st.integers(1, 4),
       W=st.integers(1, 600), price=st.sampled_from([0, 2, 4, 8, 16, 64]))
def test_pick_merge_matches_the_oracle_plan(lens, H, W, price):
    assert hd.hpc_decode_pick_merge(np.array(lens), H, W, price) is _rule(lens, H, W, price)


def test_pick_merge_errors():
    lib = hd.lib()
    lens = np.array([100, 200], dtype=np.int32)
    p = lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert lib.hpc_decode_pick_merge(p, 2, 1, 8, 0) == 1     # 6 tiles over 8 workers
    assert lib.hpc_decode_pick_merge(p, 2, 1, 4, 0) == 0     # more tiles than workers
    assert lib.hpc_decode_pick_merge(None, 2, 1, 4, 0) == hd.HPC_ERR_NULL
    assert lib.hpc_decode_pick_merge(None, 0, 1, 4, 0) == 1                  # empty batch
    assert lib.hpc_decode_pick_merge(p, -1, 1, 4, 0) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_pick_merge(p, 2, 0, 4, 0) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_pick_merge(p, 2, 1, 0, 0) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_pick_merge(p, 2, 1, 4, -1) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_pick_merge(p, 2, 1, 4, hd.MAX_ENTRY_PRICE + 1) == hd.HPC_ERR_INVALID
    bad = np.array([100, -1], dtype=np.int32)
    assert lib.hpc_decode_pick_merge(bad.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 2, 1, 4, 0) == \
        hd.HPC_ERR_INVALID
