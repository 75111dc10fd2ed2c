"""The prefill work-list planner and host checks (no GPU)."""
import ctypes

import numpy as np
import pytest

import load_balanced_paged_step_amd as hd
from load_balanced_paged_step_amd.prefill import hpc_prefill_plan, hpc_prefill_units

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


@pytest.mark.parametrize("q_lens,seq_lens,H", [
    ([512], [512], 8),
    ([1, 15, 16, 17, 0, 100], [1, 300, 16, 4000, 5, 100], 2),
    ([33] * 5, [33, 97, 64, 65, 1000], 1),
])
def test_plan_covers_every_unit_once_longest_first(q_lens, seq_lens, H):
    qs = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    work = hpc_prefill_plan(qs, seq_lens, H, max_pages_per_seq=64)
    exp = _expected_units(q_lens, seq_lens, H)
    assert hpc_prefill_units(qs, H) == len(exp) == work.shape[0]
    assert sorted(map(tuple, work.tolist())) == sorted(exp)
    cost = work[:, 3]
    assert np.all(cost[:-1] >= cost[1:])
    # ties keep (sequence, block, head) order
    for c in np.unique(cost):
        sel = work[cost == c][:, :3].tolist()
        assert sel == sorted(sel)


def test_plan_errors():
    lib = hd.lib()
    qs = np.array([0, 10, 20], dtype=np.int32)
    sl = np.array([10, 20], dtype=np.int32)
    work = np.zeros((100, 4), dtype=np.int32)
    p = lambda a: a.ctypes.data_as(I32P)
    assert lib.hpc_prefill_plan(p(qs), p(sl), 2, 1, 4, p(work), 100) == 2
    assert lib.hpc_prefill_plan(p(qs), p(sl), 2, 1, 4, p(work), 1) == hd.HPC_ERR_TOO_SMALL
    assert lib.hpc_prefill_plan(p(qs), p(np.array([9, 20], dtype=np.int32)), 2, 1, 4, p(work), 100) == hd.HPC_ERR_INVALID
    assert lib.hpc_prefill_plan(p(qs), p(sl), 2, 1, 0, p(work), 100) == hd.HPC_ERR_INVALID
    assert lib.hpc_prefill_plan(p(qs), p(np.array([10, 300], dtype=np.int32)), 2, 1, 4, p(work), 100) == hd.HPC_ERR_INVALID
    assert lib.hpc_prefill_plan(p(np.array([0, 10, 5], dtype=np.int32)), p(sl), 2, 1, 4, p(work), 100) == hd.HPC_ERR_INVALID
    assert lib.hpc_prefill_plan(p(np.array([1, 10, 20], dtype=np.int32)), p(sl), 2, 1, 4, p(work), 100) == hd.HPC_ERR_INVALID
    assert lib.hpc_prefill_plan(None, p(sl), 2, 1, 4, p(work), 100) == hd.HPC_ERR_NULL
    assert lib.hpc_prefill_units(p(qs), 0, 1) == hd.HPC_ERR_INVALID
    assert lib.hpc_prefill_units(p(qs), 2, 0) == hd.HPC_ERR_INVALID


def test_check_errors():
    lib = hd.lib()
    fake = ctypes.c_void_p(0x1000)
    ok = hd.make_params(16, 2, 8, 32, hd.HPC_KV_BF16, 0.088)
    args = lambda **kw: [kw.get(n, fake) for n in ("q", "qs", "k", "v", "bt", "sl", "work")]

    def call(params, batch=2, total=40, n_units=4, **kw):
        a = args(**kw)
        return lib.hpc_prefill_check(ctypes.byref(params), batch, total, *a, n_units, kw.get("out", fake),
                                     kw.get("lse", fake))
    assert call(ok) == hd.HPC_OK
    assert call(ok, q=None) == hd.HPC_ERR_NULL
    assert call(ok, work=None) == hd.HPC_ERR_NULL
    assert call(ok, work=None, n_units=0) == hd.HPC_OK
    assert call(ok, lse=None) == hd.HPC_ERR_NULL
    assert call(ok, batch=0) == hd.HPC_ERR_INVALID
    assert call(ok, n_units=-1) == hd.HPC_ERR_INVALID
    assert call(hd.make_params(16, 2, 8, 32, hd.HPC_KV_BF16, 0.088, head_dim=64)) == hd.HPC_ERR_UNSUPPORTED
    assert call(hd.make_params(16, 2, 8, 32, hd.HPC_KV_BF16, 0.088, tile_math="valu")) == hd.HPC_ERR_UNSUPPORTED
    assert call(hd.make_params(16, 2, 8, 32, hd.HPC_KV_BF16, 0.088, fused_merge=True)) == hd.HPC_ERR_UNSUPPORTED
    assert call(hd.make_params(64, 2, 8, 32, hd.HPC_KV_BF16, 0.088)) == hd.HPC_ERR_UNSUPPORTED     # G = 32
    assert call(hd.make_params(15, 2, 8, 32, hd.HPC_KV_BF16, 0.088)) == hd.HPC_ERR_INVALID
    assert call(hd.make_params(16, 2, 8, 32, hd.HPC_KV_BF16, float("nan"))) == hd.HPC_ERR_INVALID


def test_check_refuses_a_non_positive_score_scale():
    """The kernel keeps its running max on raw scores, so the score scale
    sm_scale * k_scale must be positive."""
    lib = hd.lib()
    fake = ctypes.c_void_p(0x1000)
    for sm, ks, code in ((0.088, 1.0, hd.HPC_OK), (-0.088, 1.0, hd.HPC_ERR_INVALID), (0.0, 1.0, hd.HPC_ERR_INVALID),
                         (0.088, -2.0, hd.HPC_ERR_INVALID)):
        p = hd.make_params(16, 2, 8, 32, hd.HPC_KV_BF16, sm, k_scale=ks)
        assert lib.hpc_prefill_check(ctypes.byref(p), 2, 40, fake, fake, fake, fake, fake, fake, fake, 4, fake,
                                     fake) == code
