"""Parity of causal prefill / extend attention (hpc_prefill_attn through the
C ABI) against the float64 oracle (oracle.prefill).

Bars, as for decode: max|out - oracle| <= 1e-2 max|V| (bf16 KV) or 3e-2
max|V| (fp8, oracle on the dequantised cache); per (query row, KV head)
unit max|out_u - oracle_u| <= 1e-2 max|oracle_u| + 1e-6 (the same bf16
roundings of P and of the output enter as in decode); |lse - oracle| <=
1e-3 (bf16) or 1e-2 (fp8).  At full size, sampled rows are checked against
the decode oracle over the row's first p + 1 tokens (the row at position p
sees exactly those), computed one row at a time.
"""
import numpy as np
import pytest
import torch

import load_balanced_paged_step_amd as hd
from load_balanced_paged_step_amd.prefill import PrefillStep
from oracle import decode_attention, prefill_attention
from workloads import make_prefill_inputs, prefill_workload_inputs

from decode_harness import LSE_TOL, OUT_TOL, WORST_UNIT, announce, max_abs_v, unit_check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hd.lib()


def run_gpu(pi, n_workers=0, min_share_tiles=1):
    """Small cases cut with no floor on the share length (min_share_tiles =
    1), so that their few tiles are still spread over several shares."""
    c = pi.cache
    q, k, v = pi.q.cuda(), c.k_cache.cuda(), c.v_cache.cuda()
    bt, sl, qs = c.block_table.cuda(), c.seq_lens.cuda(), pi.q_start.cuda()
    step = PrefillStep(pi.q_start, c.seq_lens, c.num_q_heads, c.num_kv_heads, c.max_pages_per_seq, n_workers,
                       min_share_tiles)
    if n_workers:
        assert step.n_merge > 0, "the balanced case must cut at least one unit"
    if step.workspace is not None:
        step.workspace.fill_(0xFF)          # NaN partials unless the kernel writes every slot it merges
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    step(q, qs, k, v, bt, sl, out, lse, sm_scale=c.sm_scale, k_scale=c.k_scale, v_scale=c.v_scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def run_oracle(pi):
    c = pi.cache
    return prefill_attention(pi.q_bits(), c.k_bits(), c.v_bits(), c.block_table.numpy(), c.seq_lens.numpy(),
                             pi.q_start.numpy(), num_q_heads=c.num_q_heads, num_kv_heads=c.num_kv_heads,
                             kv_format=c.kv_dtype, sm_scale=c.sm_scale, k_scale=c.k_scale, v_scale=c.v_scale)


def compare_rows(pi, got, ref, what, rows=None):
    c = pi.cache
    out, lse = got
    ref_out, ref_lse = ref
    if rows is not None:
        out, lse = out[rows], lse[rows]
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    tol = OUT_TOL[c.kv_dtype] * max_abs_v(c)
    err = float(np.abs(out - ref_out).max()) if out.size else 0.0
    assert err <= tol, f"{what}: max|out-ref| = {err:.3e} > {tol:.3e}"
    ratio, where = unit_check(out, ref_out, c.num_kv_heads, what)
    key = f"prefill {c.kv_dtype}"
    if key not in WORST_UNIT or ratio > WORST_UNIT[key][0]:
        WORST_UNIT[key] = (ratio, f"{what} {where}")
    lerr = float(np.abs(lse - ref_lse).max()) if lse.size else 0.0
    assert lerr <= LSE_TOL[c.kv_dtype], f"{what}: max|lse-ref| = {lerr:.3e}"


CASES = {
    "prompt 200, 8q/1kv": ([0], [200], 8, 1, "bf16"),
    "prompt 512, 64q/8kv": ([0], [512], 64, 8, "bf16"),
    "ragged extends, 16q/2kv": ([100, 0, 63, 1000, 5, 64], [1, 15, 17, 33, 64, 0], 16, 2, "bf16"),
    "extends G=1": ([300, 20], [40, 70], 4, 4, "bf16"),
    "extends G=2": ([128, 7], [50, 9], 8, 4, "bf16"),
    "extends G=16 (two workgroups of 8 heads)": ([70, 0], [45, 130], 32, 2, "bf16"),
    "extends G=12 (the second workgroup's heads part-filled)": ([50, 200], [70, 33], 24, 2, "bf16"),
    "extends G=5": ([90], [77], 5, 1, "bf16"),
    "extends G=3 (two heads per wave, two-wave groups)": ([150, 0], [50, 64], 6, 2, "bf16"),
    "extends G=4 (two heads per wave, two-wave groups)": ([300, 20, 0], [40, 70, 33], 16, 4, "bf16"),
    "fp8 extends G=4": ([500, 30], [64, 17], 32, 8, "fp8_e4m3"),
    "fp8 extends 64q/8kv": ([2000, 64, 0], [256, 100, 65], 64, 8, "fp8_e4m3"),
    "fp8 prompt G=16": ([0], [300], 16, 1, "fp8_e4m3"),
    "one-token chunks (decode)": ([37, 64, 3000], [1, 1, 1], 8, 1, "bf16"),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_prefill_parity(case):
    ctx, n, hq, hkv, kv = CASES[case]
    announce(f"prefill parity, {case}")
    pi = make_prefill_inputs(ctx, n, hq, hkv, kv, seed=sum(ctx) + sum(n) + hq, poison=True)
    compare_rows(pi, run_gpu(pi), run_oracle(pi), case)


# balanced plans: long units cut into shares merged by log-sum-exp
BALANCED = {
    "prompt 200 on 64 workers, 8q/1kv": ([0], [200], 8, 1, "bf16", 64),
    "extend after 3000, 16q/2kv, 40 workers": ([3000, 0, 10], [40, 17, 1], 16, 2, "bf16", 40),
    "extends G=16 (two workgroups of 8 heads), 30 workers": ([700, 0], [45, 130], 32, 2, "bf16", 30),
    "extend G=5, one tile a share": ([300], [20], 5, 1, "bf16", 10000),
    "extends G=4 after 2000, 40 workers": ([2000, 10], [33, 20], 8, 2, "bf16", 40),
    "fp8 extends 64q/8kv, 512 workers": ([2000, 64, 0], [256, 100, 65], 64, 8, "fp8_e4m3", 512),
    "decode rows after 5000, 8q/1kv, 30 workers": ([5000, 37, 900], [1, 1, 1], 8, 1, "bf16", 30),
    "empty chunks and an empty sequence, G = 2 (one head per wave)": ([900, 5, 0, 40], [20, 0, 0, 33], 8, 4,
                                                                     "bf16", 100),
    # 33 one-tile shares: three merge chunks, the last holding only tile 32,
    # which rows 0..7 (positions 2040..2047) do not see
    "33 one-tile shares, a chunk with no visible token": ([2040], [16], 8, 1, "bf16", 10000),
}


@pytest.mark.parametrize("case", sorted(BALANCED))
def test_balanced_prefill_parity(case):
    ctx, n, hq, hkv, kv, W = BALANCED[case]
    announce(f"balanced prefill parity, {case}")
    pi = make_prefill_inputs(ctx, n, hq, hkv, kv, seed=sum(ctx) + sum(n) + hq + 1, poison=True)
    compare_rows(pi, run_gpu(pi, W), run_oracle(pi), f"balanced {case}")


def test_balanced_and_whole_units_agree():
    """Cut and uncut plans of the same extend: the shares' merge changes
    only rounding (partials merged in fp32, one bf16 rounding of out)."""
    pi = make_prefill_inputs([2500, 100], [64, 33], 16, 2, "bf16", seed=12)
    announce("balanced vs whole units")
    a, b = run_gpu(pi), run_gpu(pi, 64)
    tol = OUT_TOL["bf16"] * max_abs_v(pi.cache)
    assert float(np.abs(a[0] - b[0]).max()) <= tol
    assert float(np.abs(a[1] - b[1]).max()) <= LSE_TOL["bf16"]


@pytest.mark.parametrize("name", ["prefill-q512", "prefill-q512-8q1kv"])
def test_prompt_workloads_full(name):
    announce(f"prefill workload {name}, every row")
    pi = prefill_workload_inputs(name, poison=True)
    compare_rows(pi, run_gpu(pi), run_oracle(pi), name)


@pytest.mark.parametrize("name,n_workers", [("extend-8x512", 0), ("extend-8x256-fp8", 0), ("extend-8x256-fp8", 1024),
                                            ("extend-32k+512-8q1kv", 512), ("extend-128k+7x4k-8q1kv", 512)])
def test_extend_workloads_sampled(name, n_workers):
    """Full-size extend batches, whole units or balanced (cut units in each):
    96 sampled rows, each against the decode oracle over that row's visible
    prefix."""
    announce(f"prefill workload {name}, n_workers {n_workers}, sampled rows")
    _check_sampled(prefill_workload_inputs(name, poison=True), n_workers, f"{name} W={n_workers}")


@pytest.mark.parametrize("hq", [8, 16, 32])
def test_small_groups_on_a_full_grid(hq):
    """extend-8x512's contexts and chunks with 8 KV heads and 1, 2 or 4 query
    heads each: 2048 units, enough two-wave workgroups for one group each
    (the small cases above run two groups per workgroup); sampled rows."""
    from workloads import PREFILL_WORKLOADS, draw_loguniform_lengths
    w = PREFILL_WORKLOADS["extend-8x512"]
    rng = np.random.default_rng(7)
    ctx = draw_loguniform_lengths(rng, len(w.q_lens), *w.ctx_loguniform)
    announce(f"prefill extend-8x512 contexts, {hq}q/8kv, sampled rows")
    pi = make_prefill_inputs(ctx, w.q_lens, hq, 8, "bf16", seed=7, poison=True)
    _check_sampled(pi, 0, f"extend-8x512 contexts {hq}q/8kv")


def _check_sampled(pi, n_workers, what):
    c = pi.cache
    got = run_gpu(pi, n_workers, PrefillStep.MIN_SHARE_TILES)
    rng = np.random.default_rng(11)
    qs = pi.q_start.numpy()
    rows = np.sort(rng.choice(pi.total, size=96, replace=False))
    # always include every sequence's first and last row
    rows = np.unique(np.concatenate([rows, qs[:-1], qs[1:] - 1]))
    ref_out = np.zeros((rows.size, c.num_q_heads, 128))
    ref_lse = np.zeros((rows.size, c.num_q_heads))
    for i, r in enumerate(rows):
        b = int(np.searchsorted(qs, r, side="right") - 1)
        n, L = qs[b + 1] - qs[b], int(c.seq_lens[b])
        p = L - n + (r - qs[b])
        o, l = decode_attention(pi.q_bits()[r:r + 1], c.k_bits(), c.v_bits(), c.block_table.numpy()[b:b + 1],
                                np.array([p + 1]), num_q_heads=c.num_q_heads, num_kv_heads=c.num_kv_heads,
                                kv_format=c.kv_dtype, sm_scale=c.sm_scale, k_scale=c.k_scale, v_scale=c.v_scale)
        ref_out[i], ref_lse[i] = o[0], l[0]
    compare_rows(pi, got, (ref_out, ref_lse), what, rows=rows)


@pytest.mark.parametrize("n_workers", [0, 48])
def test_bitwise_deterministic_and_page_permutation(n_workers):
    pi = make_prefill_inputs([700, 65], [130, 64], 16, 2, "bf16", seed=5)
    announce(f"prefill determinism and page permutation, n_workers {n_workers}")
    a = run_gpu(pi, n_workers)
    b = run_gpu(pi, n_workers)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = pi.cache
    perm = np.random.default_rng(3).permutation(c.num_pages)
    k, v = torch.empty_like(c.k_cache), torch.empty_like(c.v_cache)
    k[torch.from_numpy(perm)] = c.k_cache
    v[torch.from_numpy(perm)] = c.v_cache
    c.k_cache, c.v_cache = k, v
    c.block_table = torch.from_numpy(perm[c.block_table.numpy()].astype(np.int32))
    p = run_gpu(pi, n_workers)
    assert np.array_equal(a[0], p[0]) and np.array_equal(a[1], p[1])


def test_first_row_of_a_prompt_is_v0():
    pi = make_prefill_inputs([0], [40], 8, 1, "bf16", seed=6)
    announce("prefill first row = V_0")
    out, lse = run_gpu(pi)
    c = pi.cache
    v0 = c.v_cache[int(c.block_table[0, 0]), 0, 0].float().numpy()
    for hq in range(8):
        assert np.array_equal(out[0, hq], v0)      # one visible token: P = 1 exactly, out = bf16(V_0)
