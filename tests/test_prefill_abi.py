"""The prefill work-list planner and host checks (no GPU)."""
import ctypes

import numpy as np
import pytest

import load_balanced_paged_step_amd as hd
from load_balanced_paged_step_amd.prefill import (hpc_prefill_plan, hpc_prefill_plan_size, hpc_prefill_units,
                                                  hpc_prefill_workspace_size)

I32P = ctypes.POINTER(ctypes.c_int32)


def _expected_units(q_lens, seq_lens, H):
    """Every (sequence, 16-query block, KV head) with the number of 64-token
    tiles its last query sees, from the definition of the positions."""
    out = []
    for b, (n, L) in enumerate(zip(q_lens, seq_lens)):
        for j in range((n + 15) // 16):
            last_query = min(16 * (j + 1), n) - 1
            p = L - n + last_query
            for h in range(H):
                out.append((b, j, h, p // 64 + 1))
    return out


def _plan(q_lens, seq_lens, H, n_workers=0, max_pages=64, min_share=1):
    qs = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    words, counts = hpc_prefill_plan(qs, seq_lens, H, max_pages_per_seq=max_pages, n_workers=n_workers,
                                     min_share_tiles=min_share)
    n_e, n_m, n_p = counts
    assert words.size == 8 * n_e + 8 * n_m <= hpc_prefill_plan_size(qs, H, n_workers)
    return qs, words[:8 * n_e].reshape(-1, 8), words[8 * n_e:].reshape(-1, 8), n_p


@pytest.mark.parametrize("q_lens,seq_lens,H", [
    ([512], [512], 8),
    ([1, 15, 16, 17, 0, 100], [1, 300, 16, 4000, 5, 100], 2),
    ([33] * 5, [33, 97, 64, 65, 1000], 1),
])
def test_plan_covers_every_unit_once_longest_first(q_lens, seq_lens, H):
    qs, ent, merge, n_p = _plan(q_lens, seq_lens, H)
    exp = _expected_units(q_lens, seq_lens, H)
    assert hpc_prefill_units(qs, H) == len(exp) == ent.shape[0]
    assert merge.shape[0] == 0 and n_p == 0
    assert sorted(map(tuple, ent[:, :4].tolist())) == sorted(exp)
    assert np.all(ent[:, 4] == 0) and np.all(ent[:, 5] == ent[:, 3]) and np.all(ent[:, 6] == -1)
    assert np.all(ent[:, 7] == 0)
    cost = ent[:, 3]
    assert np.all(cost[:-1] >= cost[1:])
    # ties keep (sequence, block, head) order
    for c in np.unique(cost):
        sel = ent[cost == c][:, :3].tolist()
        assert sel == sorted(sel)


@pytest.mark.parametrize("q_lens,seq_lens,H,W,min_share", [
    ([512], [32768 + 512], 1, 256, 1),                 # one long extend, 8 q / 1 kv: 32 very long units
    ([512], [32768 + 512], 1, 256, 100),               # ... with shares of at least 100 tiles
    ([16, 512, 1], [70000, 512, 9000], 2, 100, 1),
    ([512], [512], 8, 256, 1),                         # a prompt: units of 1..8 tiles, the longest cut
    ([512], [512], 8, 256, 16),                        # ... and none with a 16-tile floor
    ([1, 15, 16, 17, 0, 100], [1, 300, 16, 4000, 5, 100], 2, 7, 3),
    ([64], [64 * 64], 1, 1, 1),                        # one worker: nothing is cut (q = T)
    ([64, 64], [64 * 100, 64 * 30], 1, 4, 1),          # T/W ~ 130/4: the 100-tile units cut, the 30-tile kept
    ([3, 3], [64 * 40, 5], 1, 10000, 1),               # more workers than tiles: q = 1, one tile a share
])
def test_balanced_plan_cuts_long_units_at_multiples_of_q(q_lens, seq_lens, H, W, min_share):
    """With W workers and q = max(ceil(T / W), min_share), a unit of n > 2 q
    tiles is S = ceil(n / q) shares [k q, min((k+1) q, n)) with partial slots
    base .. base + S - 1, a unit of n <= 2 q one entry; every tile of every
    unit covered once, every slot written once; entries longest first, ties
    by first tile then unit order."""
    qs, ent, merge, n_p = _plan(q_lens, seq_lens, H, W, max_pages=2048, min_share=min_share)
    units = _expected_units(q_lens, seq_lens, H)
    T = sum(u[3] for u in units)
    q = max(1, -(-T // W), min_share)
    assert np.all(ent[:, 3] <= 2 * q) and np.all(ent[:, 3] == ent[:, 5] - ent[:, 4]) and np.all(ent[:, 3] >= 1)
    assert np.all(ent[ent[:, 6] >= 0, 3] <= q)
    order = {u[:3]: i for i, u in enumerate(units)}
    keys = [(-e[3], e[4], order[tuple(e[:3])]) for e in ent.tolist()]
    assert keys == sorted(keys)
    by_unit = {}
    for e in ent.tolist():
        by_unit.setdefault(tuple(e[:3]), []).append(e)
    assert sorted(by_unit) == sorted(u[:3] for u in units)
    merged = {tuple(m[:3]): m for m in merge.tolist()}
    base_expected = 0
    for (b, j, h, n) in units:                          # unit order numbers the slots
        shares = sorted(by_unit[(b, j, h)], key=lambda e: e[4])
        S = -(-n // q) if n > 2 * q else 1
        assert len(shares) == S
        if S == 1:
            assert shares[0][4:7] == [0, n, -1] and (b, j, h) not in merged
            continue
        assert [(e[4], e[5]) for e in shares] == [(k * q, min((k + 1) * q, n)) for k in range(S)]
        assert [e[6] for e in shares] == list(range(base_expected, base_expected + S))
        assert merged[(b, j, h)] == [b, j, h, S, base_expected, 0, 0, 0]
        base_expected += S
    assert n_p == base_expected
    assert [tuple(m[:3]) for m in merge.tolist()] == [u[:3] for u in units if u[3] > 2 * q]
    assert ent.shape[0] <= len(units) + W


def test_balanced_plan_of_one_long_extend_fills_the_workers():
    """8 query heads on one KV head, 512 new tokens after 32K cached: 32 units
    of about 520 tiles.  Unbalanced, 32 workgroups carry everything; with 256
    workers no entry is longer than ceil(T / 256)."""
    _, ent0, _, _ = _plan([512], [32768 + 512], 1, 0, max_pages=1024)
    _, ent, merge, n_p = _plan([512], [32768 + 512], 1, 256, max_pages=1024)
    T = int(ent0[:, 3].sum())
    assert ent0.shape[0] == 32 and int(ent[:, 3].sum()) == T
    assert ent.shape[0] >= 256 and ent[:, 3].max() <= -(-T // 256)
    assert merge.shape[0] == 32 and n_p == ent.shape[0]


def test_plan_errors():
    lib = hd.lib()
    qs = np.array([0, 10, 20], dtype=np.int32)
    sl = np.array([10, 20], dtype=np.int32)
    work = np.zeros(800, dtype=np.int32)
    counts = np.zeros(3, dtype=np.int32)
    p = lambda a: a.ctypes.data_as(I32P)
    plan = lambda qs_, sl_, mp=4, W=0, cap=800, cnt=counts, ms=1: lib.hpc_prefill_plan(
        p(qs_) if qs_ is not None else None, p(sl_), 2, 1, mp, W, ms, p(work), cap, p(cnt) if cnt is not None else None)
    assert plan(qs, sl) == hd.HPC_OK and list(counts) == [2, 0, 0]
    assert plan(qs, sl, cap=15) == hd.HPC_ERR_TOO_SMALL
    assert plan(qs, sl, cap=16) == hd.HPC_OK
    assert plan(qs, sl, W=-1) == hd.HPC_ERR_INVALID
    assert plan(qs, sl, ms=0) == hd.HPC_ERR_INVALID
    assert plan(qs, sl, cnt=None) == hd.HPC_ERR_NULL
    assert plan(qs, np.array([9, 20], dtype=np.int32)) == hd.HPC_ERR_INVALID
    assert plan(qs, sl, mp=0) == hd.HPC_ERR_INVALID
    assert plan(qs, np.array([10, 300], dtype=np.int32)) == hd.HPC_ERR_INVALID
    assert plan(np.array([0, 10, 5], dtype=np.int32), sl) == hd.HPC_ERR_INVALID
    assert plan(np.array([1, 10, 20], dtype=np.int32), sl) == hd.HPC_ERR_INVALID
    assert plan(None, sl) == hd.HPC_ERR_NULL
    assert lib.hpc_prefill_units(p(qs), 0, 1) == hd.HPC_ERR_INVALID
    assert lib.hpc_prefill_units(p(qs), 2, 0) == hd.HPC_ERR_INVALID
    assert lib.hpc_prefill_plan_size(p(qs), 2, 1, -1) == hd.HPC_ERR_INVALID
    assert lib.hpc_prefill_plan_size(p(qs), 2, 1, 5) == 8 * (2 + 5) + 8 * 2


def test_workspace_size():
    assert hpc_prefill_workspace_size(0, 16, 2) == 0
    # 3 slots x 16 rows x G=8 heads: 384 fp32 rows of 128, then 384 lse after 256-byte alignment
    assert hpc_prefill_workspace_size(3, 16, 2) == 384 * 128 * 4 + 384 * 4
    assert hpc_prefill_workspace_size(1, 5, 1) == (80 * 512 + 255) // 256 * 256 + 80 * 4
    for bad in ((-1, 16, 2), (1, 16, 0), (1, 15, 2), (1, 1, 2)):
        with pytest.raises(RuntimeError):
            hpc_prefill_workspace_size(*bad)


def _check(lib, params, batch=2, total=40, n_entries=4, n_merge=0, n_partials=0, ws_bytes=0, **kw):
    fake = ctypes.c_void_p(0x1000)
    a = [kw.get(n, fake) for n in ("q", "qs", "k", "v", "bt", "sl", "work")]
    return lib.hpc_prefill_check(ctypes.byref(params), batch, total, *a, n_entries, n_merge, n_partials,
                                 kw.get("ws", fake), ws_bytes, kw.get("out", fake), kw.get("lse", fake))


def test_check_errors():
    lib = hd.lib()
    ok = hd.make_params(16, 2, 8, 32, hd.HPC_KV_BF16, 0.088)
    call = lambda params, **kw: _check(lib, params, **kw)
    assert call(ok) == hd.HPC_OK
    assert call(ok, q=None) == hd.HPC_ERR_NULL
    assert call(ok, work=None) == hd.HPC_ERR_NULL
    assert call(ok, work=None, n_entries=0) == hd.HPC_OK
    assert call(ok, lse=None) == hd.HPC_ERR_NULL
    assert call(ok, batch=0) == hd.HPC_ERR_INVALID
    assert call(ok, n_entries=-1) == hd.HPC_ERR_INVALID
    assert call(hd.make_params(16, 2, 8, 32, hd.HPC_KV_BF16, 0.088, head_dim=64)) == hd.HPC_ERR_UNSUPPORTED
    assert call(hd.make_params(16, 2, 8, 32, hd.HPC_KV_BF16, 0.088, tile_math="valu")) == hd.HPC_ERR_UNSUPPORTED
    assert call(hd.make_params(16, 2, 8, 32, hd.HPC_KV_BF16, 0.088, fused_merge=True)) == hd.HPC_ERR_UNSUPPORTED
    assert call(hd.make_params(64, 2, 8, 32, hd.HPC_KV_BF16, 0.088)) == hd.HPC_ERR_UNSUPPORTED     # G = 32
    assert call(hd.make_params(15, 2, 8, 32, hd.HPC_KV_BF16, 0.088)) == hd.HPC_ERR_INVALID
    assert call(hd.make_params(16, 2, 8, 32, hd.HPC_KV_BF16, float("nan"))) == hd.HPC_ERR_INVALID
    # the partials' workspace and the plan's counts
    need = hpc_prefill_workspace_size(5, 16, 2)
    cut = dict(n_entries=8, n_merge=2, n_partials=5)
    assert call(ok, ws_bytes=need, **cut) == hd.HPC_OK
    assert call(ok, ws_bytes=need - 1, **cut) == hd.HPC_ERR_TOO_SMALL
    assert call(ok, ws_bytes=need, ws=None, **cut) == hd.HPC_ERR_NULL
    assert call(ok, ws=None) == hd.HPC_OK                              # no partials, no workspace
    assert call(ok, n_entries=8, n_merge=2, n_partials=0) == hd.HPC_ERR_PLAN_MISMATCH
    assert call(ok, n_entries=8, n_merge=0, n_partials=3, ws_bytes=need) == hd.HPC_ERR_PLAN_MISMATCH
    # every cut unit has at least two shares, each an entry
    assert call(ok, n_entries=8, n_merge=3, n_partials=5, ws_bytes=need) == hd.HPC_ERR_PLAN_MISMATCH
    assert call(ok, n_entries=4, n_merge=2, n_partials=5, ws_bytes=need) == hd.HPC_ERR_PLAN_MISMATCH
    assert call(ok, n_merge=-1) == hd.HPC_ERR_INVALID


def test_check_refuses_a_non_positive_score_scale():
    """The kernel keeps its running max on raw scores, so the score scale
    sm_scale * k_scale must be positive."""
    lib = hd.lib()
    for sm, ks, code in ((0.088, 1.0, hd.HPC_OK), (-0.088, 1.0, hd.HPC_ERR_INVALID), (0.0, 1.0, hd.HPC_ERR_INVALID),
                         (0.088, -2.0, hd.HPC_ERR_INVALID)):
        p = hd.make_params(16, 2, 8, 32, hd.HPC_KV_BF16, sm, k_scale=ks)
        assert _check(lib, p) == code
