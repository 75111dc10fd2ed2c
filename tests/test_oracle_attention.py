"""Pins for oracle.attention: brute force, closed forms and invariants.

None of these re-types the oracle's formula: the brute force goes through
torch's float64 scaled_dot_product_attention on contiguous K/V gathered by a
loop written here, the closed forms are solved by hand, and the invariants
(page permutation, split / merge) hold for any correct implementation.
"""
import math

import numpy as np
import pytest
import torch

from oracle.attention import (decode_attention, merge_partials, range_attention,
                              split_decode_attention)
from oracle.formats import bf16_bits_to_f64
from workloads import make_inputs, PAGE

SM = 1.0 / math.sqrt(128)


def _run(inp, **kw):
    return decode_attention(inp.q_bits(), inp.k_bits(), inp.v_bits(), inp.block_table.numpy(),
                            inp.seq_lens.numpy(), num_q_heads=inp.num_q_heads,
                            num_kv_heads=inp.num_kv_heads, kv_format=inp.kv_dtype,
                            sm_scale=kw.get("sm_scale", inp.sm_scale), k_scale=inp.k_scale,
                            v_scale=inp.v_scale)


def _dense_reference(inp):
    """Gather each sequence into contiguous K/V with plain loops, then SDPA in float64."""
    B, Hq, D = inp.q.shape
    G = Hq // inp.num_kv_heads
    k = inp.k_cache.to(torch.float64) * inp.k_scale
    v = inp.v_cache.to(torch.float64) * inp.v_scale
    q = inp.q.to(torch.float64)
    out = torch.zeros(B, Hq, D, dtype=torch.float64)
    lse = torch.full((B, Hq), -math.inf, dtype=torch.float64)
    for b in range(B):
        L = int(inp.seq_lens[b])
        if L == 0:
            continue
        rows_k, rows_v = [], []
        for t in range(L):
            pg = int(inp.block_table[b, t // PAGE])
            rows_k.append(k[pg, :, t % PAGE, :])
            rows_v.append(v[pg, :, t % PAGE, :])
        K = torch.stack(rows_k, dim=1)            # [H_kv, L, D]
        V = torch.stack(rows_v, dim=1)
        for hq in range(Hq):
            h = hq // G
            o = torch.nn.functional.scaled_dot_product_attention(
                q[b, hq][None, None, None, :], K[h][None, None], V[h][None, None], scale=inp.sm_scale)
            out[b, hq] = o[0, 0, 0]
            s = (K[h] @ q[b, hq]) * inp.sm_scale
            lse[b, hq] = torch.logsumexp(s, dim=0)
    return out.numpy(), lse.numpy()


@pytest.mark.parametrize("lens,hq,hkv,fmt", [
    ([37, 64, 130, 200], 8, 1, "bf16"),
    ([1, 65, 3], 4, 2, "bf16"),
    ([0, 129, 17], 8, 1, "bf16"),
    ([70, 5], 16, 2, "fp8_e4m3"),
    ([200, 64, 1], 8, 4, "fp8_e4m3"),
])
def test_matches_dense_brute_force(lens, hq, hkv, fmt):
    inp = make_inputs(lens, hq, hkv, fmt, seed=sum(lens) + hq)
    out, lse = _run(inp)
    ref_out, ref_lse = _dense_reference(inp)
    np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_single_token_returns_v0_exactly():
    inp = make_inputs([1, 1], 8, 2, "bf16", seed=3)
    out, lse = _run(inp)
    for b in range(2):
        pg = int(inp.block_table[b, 0])
        for hq in range(8):
            h = hq // 4
            v0 = bf16_bits_to_f64(inp.v_bits()[pg, h, 0])
            assert np.array_equal(out[b, hq], v0)
            k0 = bf16_bits_to_f64(inp.k_bits()[pg, h, 0])
            q = bf16_bits_to_f64(inp.q_bits()[b, hq])
            assert lse[b, hq] == pytest.approx(SM * float(q @ k0), rel=1e-15, abs=1e-15)


def test_identical_keys_give_mean_of_values():
    L = 150
    inp = make_inputs([L], 8, 1, "bf16", seed=4)
    k = inp.k_cache.view(torch.int16)
    k[:] = k[int(inp.block_table[0, 0]), 0, 0]          # every row = the same key
    out, lse = _run(inp)
    V = np.stack([bf16_bits_to_f64(inp.v_bits()[int(inp.block_table[0, t // PAGE]), 0, t % PAGE])
                  for t in range(L)])
    np.testing.assert_allclose(out[0], np.broadcast_to(V.mean(axis=0), (8, 128)), rtol=0, atol=1e-13)
    key = bf16_bits_to_f64(inp.k_bits()[0, 0, 0])
    for hq in range(8):
        s = SM * float(bf16_bits_to_f64(inp.q_bits()[0, hq]) @ key)
        assert lse[0, hq] == pytest.approx(s + math.log(L), rel=1e-13)


def test_constant_values_give_that_constant():
    inp = make_inputs([300, 7], 8, 1, "bf16", seed=5)
    inp.v_cache.view(torch.int16).fill_(0x3FC0)            # bf16 1.5
    out, _ = _run(inp)
    np.testing.assert_allclose(out, 1.5, rtol=0, atol=1e-14)


def test_needle_key_dominates():
    L = 500
    inp = make_inputs([L], 8, 1, "bf16", seed=6)
    inp.q.fill_(1.0)
    inp.k_cache.fill_(0.0)
    needle = 321
    pg = int(inp.block_table[0, needle // PAGE])
    inp.k_cache[pg, 0, needle % PAGE, :] = 8.0              # s = 128*8/sqrt(128) ~ 90.5
    out, _ = _run(inp)
    vn = inp.v_cache[pg, 0, needle % PAGE].to(torch.float64).numpy()
    np.testing.assert_allclose(out[0], np.broadcast_to(vn, (8, 128)), rtol=0, atol=1e-30)


def test_two_token_hand_solved():
    """q = 8 e0, k0 = 0, k1 = 2 e0  =>  s0 = 0, s1 = 16/sqrt(128) = sqrt(2).

    out = (v0 + e^sqrt2 v1) / (1 + e^sqrt2),  lse = ln(1 + e^sqrt2).
    """
    inp = make_inputs([2], 8, 1, "bf16", seed=7)
    inp.q.zero_()
    inp.q[0, :, 0] = 8.0
    pg = int(inp.block_table[0, 0])
    inp.k_cache[pg, 0, 0] = 0.0
    inp.k_cache[pg, 0, 1] = 0.0
    inp.k_cache[pg, 0, 1, 0] = 2.0
    inp.v_cache[pg, 0, 0] = 0.0
    inp.v_cache[pg, 0, 1] = 0.0
    inp.v_cache[pg, 0, 0, 5] = 1.0
    inp.v_cache[pg, 0, 1, 5] = -3.0
    inp.v_cache[pg, 0, 1, 9] = 0.5
    out, lse = _run(inp)
    e = math.exp(math.sqrt(2.0))
    expect = np.zeros(128)
    expect[5] = (1.0 - 3.0 * e) / (1.0 + e)
    expect[9] = 0.5 * e / (1.0 + e)
    for hq in range(8):
        np.testing.assert_allclose(out[0, hq], expect, rtol=1e-14, atol=1e-15)
        assert lse[0, hq] == pytest.approx(math.log1p(e), rel=1e-14)


def test_empty_sequence():
    inp = make_inputs([0, 5], 8, 1, "bf16", seed=8)
    out, lse = _run(inp)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(out[1])) and np.all(np.isfinite(lse[1]))


@pytest.mark.parametrize("fmt", ["bf16", "fp8_e4m3"])
def test_page_permutation_is_bitwise_invariant(fmt):
    inp = make_inputs([100, 257, 64, 3], 8, 2, fmt, seed=9)
    out, lse = _run(inp)
    rng = np.random.default_rng(99)
    n = inp.num_pages
    perm = rng.permutation(n)                 # new position of old page i is perm[i]
    new_k = torch.empty_like(inp.k_cache)
    new_v = torch.empty_like(inp.v_cache)
    new_k[torch.from_numpy(perm)] = inp.k_cache
    new_v[torch.from_numpy(perm)] = inp.v_cache
    inp.k_cache, inp.v_cache = new_k, new_v
    inp.block_table = torch.from_numpy(perm[inp.block_table.numpy()].astype(np.int32))
    out2, lse2 = _run(inp)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_poisoned_tails_and_padding_are_never_read():
    a = make_inputs([37, 130, 1], 8, 1, "bf16", seed=10, poison=False)
    b = make_inputs([37, 130, 1], 8, 1, "bf16", seed=10, poison=True)
    oa, la = _run(a)
    ob, lb = _run(b)
    assert np.all(np.isfinite(ob)) and np.array_equal(oa, ob) and np.array_equal(la, lb)


@pytest.mark.parametrize("seed", range(6))
def test_split_and_merge_equal_unsplit(seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 700, size=3).tolist()
    hkv = int(rng.integers(1, 3))
    inp = make_inputs(lens, 4 * hkv, hkv, "bf16" if seed % 2 else "fp8_e4m3", seed=seed)
    out, lse = _run(inp)
    entries = []
    for b, L in enumerate(lens):
        n = (L + PAGE - 1) // PAGE
        for h in range(hkv):
            u = b * hkv + h
            cuts = sorted(set([0, n] + rng.integers(0, n + 1, size=3).tolist())) if n else [0, 0]
            for a, c in zip(cuts[:-1], cuts[1:]):
                if c > a:
                    entries.append((u, a, c))
    out2, lse2, parts = split_decode_attention(
        inp.q_bits(), inp.k_bits(), inp.v_bits(), inp.block_table.numpy(), inp.seq_lens.numpy(),
        entries, num_q_heads=inp.num_q_heads, num_kv_heads=hkv, kv_format=inp.kv_dtype,
        sm_scale=inp.sm_scale, k_scale=inp.k_scale, v_scale=inp.v_scale)
    assert len(parts) == len(entries)
    nonempty = np.array([L > 0 for L in lens]).repeat(inp.num_q_heads)
    np.testing.assert_allclose(out2.reshape(-1, 128)[nonempty], out.reshape(-1, 128)[nonempty],
                               rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2.reshape(-1)[nonempty], lse.reshape(-1)[nonempty], rtol=1e-12)


def test_merge_is_order_free_and_ignores_empty_parts():
    rng = np.random.default_rng(11)
    parts = [(rng.standard_normal((8, 128)), rng.standard_normal(8) * 3) for _ in range(5)]
    o1, l1 = merge_partials(parts)
    o2, l2 = merge_partials(parts[::-1] + [(np.zeros((8, 128)), np.full(8, -np.inf))])
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-14)
    # merging two halves of one sequence by hand: weights e^{lse_i}
    o, l = merge_partials(parts[:2])
    w0, w1 = np.exp(parts[0][1]), np.exp(parts[1][1])
    np.testing.assert_allclose(o, (w0[:, None] * parts[0][0] + w1[:, None] * parts[1][0])
                               / (w0 + w1)[:, None], rtol=1e-12)
    np.testing.assert_allclose(l, np.log(w0 + w1), rtol=1e-13)


def test_range_attention_of_empty_range():
    inp = make_inputs([10], 8, 1, "bf16", seed=12)
    o, l = range_attention(inp.q_bits(), inp.k_bits(), inp.v_bits(), inp.block_table.numpy(), 0, 0,
                           5, 5, num_q_heads=8, num_kv_heads=1, sm_scale=SM)
    assert np.all(o == 0) and np.all(np.isneginf(l))
