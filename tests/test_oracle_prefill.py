"""Pins for oracle.prefill (causal prefill / extend attention over pages).

The brute force goes through torch's float64 scaled_dot_product_attention
on contiguous K/V gathered token by token here (is_causal for prefill, an
explicit boolean mask for extend, whose causal diagonal sits at the bottom
right); the decode oracle (pinned on its own) must agree for chunks of one
token and for the last query of every chunk; query 0 of a prompt sees one
token, so it returns V_0 exactly.
"""
import math

import numpy as np
import pytest
import torch

from oracle.attention import decode_attention
from oracle.prefill import prefill_attention
from workloads import PAGE, make_prefill_inputs


def _run(pi):
    c = pi.cache
    return prefill_attention(pi.q_bits(), c.k_bits(), c.v_bits(), c.block_table.numpy(), c.seq_lens.numpy(),
                             pi.q_start.numpy(), num_q_heads=c.num_q_heads, num_kv_heads=c.num_kv_heads,
                             kv_format=c.kv_dtype, sm_scale=c.sm_scale, k_scale=c.k_scale, v_scale=c.v_scale)


def _gather(pi, b):
    """Contiguous K/V [H_kv, L, D] of sequence b, gathered token by token."""
    c = pi.cache
    L = int(c.seq_lens[b])
    k = c.k_cache.to(torch.float64) * c.k_scale
    v = c.v_cache.to(torch.float64) * c.v_scale
    K = torch.stack([k[int(c.block_table[b, t // PAGE]), :, t % PAGE] for t in range(L)], dim=1)
    V = torch.stack([v[int(c.block_table[b, t // PAGE]), :, t % PAGE] for t in range(L)], dim=1)
    return K, V


def _sdpa_reference(pi):
    c = pi.cache
    G = c.num_q_heads // c.num_kv_heads
    q = pi.q.to(torch.float64)
    out = torch.zeros(q.shape, dtype=torch.float64)
    s0 = pi.q_start.numpy()
    for b in range(c.batch):
        r0, r1 = int(s0[b]), int(s0[b + 1])
        n, L = r1 - r0, int(c.seq_lens[b])
        if n == 0:
            continue
        K, V = _gather(pi, b)
        K, V = K.repeat_interleave(G, dim=0), V.repeat_interleave(G, dim=0)      # [Hq, L, D]
        qb = q[r0:r1].transpose(0, 1)                                           # [Hq, n, D]
        if n == L:
            o = torch.nn.functional.scaled_dot_product_attention(qb, K, V, is_causal=True, scale=c.sm_scale)
        else:
            mask = torch.arange(L)[None, :] <= (L - n + torch.arange(n))[:, None]
            o = torch.nn.functional.scaled_dot_product_attention(qb, K, V, attn_mask=mask, scale=c.sm_scale)
        out[r0:r1] = o.transpose(0, 1)
    return out.numpy()


@pytest.mark.parametrize("ctx,n,hq,hkv,kv", [
    ([0], [200], 8, 1, "bf16"),                 # a prompt: causal from token 0
    ([0, 0], [64, 17], 16, 2, "bf16"),
    ([100, 0, 63], [30, 65, 1], 8, 2, "bf16"),  # extend: chunks after cached prefixes
    ([70, 5], [40, 3], 4, 4, "fp8_e4m3"),
])
def test_matches_torch_sdpa(ctx, n, hq, hkv, kv):
    pi = make_prefill_inputs(ctx, n, hq, hkv, kv, seed=sum(ctx) + sum(n))
    out, lse = _run(pi)
    np.testing.assert_allclose(out, _sdpa_reference(pi), rtol=1e-11, atol=1e-12)


def test_one_token_chunks_equal_decode():
    pi = make_prefill_inputs([37, 64, 300, 0], [1, 1, 1, 1], 16, 2, "bf16", seed=3)
    c = pi.cache
    out, lse = _run(pi)
    ref_out, ref_lse = decode_attention(pi.q_bits(), c.k_bits(), c.v_bits(), c.block_table.numpy(),
                                        c.seq_lens.numpy(), num_q_heads=16, num_kv_heads=2, kv_format="bf16",
                                        sm_scale=c.sm_scale)
    np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12)


def test_last_query_of_each_chunk_equals_decode():
    pi = make_prefill_inputs([0, 500, 90], [128, 33, 64], 8, 1, "bf16", seed=4)
    c = pi.cache
    out, lse = _run(pi)
    last = pi.q_start.numpy()[1:] - 1
    q_last = pi.q_bits()[last]
    ref_out, ref_lse = decode_attention(q_last, c.k_bits(), c.v_bits(), c.block_table.numpy(), c.seq_lens.numpy(),
                                        num_q_heads=8, num_kv_heads=1, kv_format="bf16", sm_scale=c.sm_scale)
    np.testing.assert_allclose(out[last], ref_out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[last], ref_lse, rtol=1e-12)


def test_first_query_of_a_prompt_returns_v0():
    pi = make_prefill_inputs([0], [50], 8, 2, "bf16", seed=5)
    out, lse = _run(pi)
    K, V = _gather(pi, 0)
    G = 4
    for hq in range(8):
        assert np.array_equal(out[0, hq], V[hq // G, 0].numpy())
        s0 = float(pi.q[0, hq].double() @ K[hq // G, 0]) * pi.cache.sm_scale
        assert math.isclose(lse[0, hq], s0, rel_tol=1e-14, abs_tol=1e-14)


def test_page_permutation_invariant():
    pi = make_prefill_inputs([200, 10], [100, 70], 8, 1, "bf16", seed=6)
    a = _run(pi)
    c = pi.cache
    perm = np.random.default_rng(1).permutation(c.num_pages)
    k, v = torch.empty_like(c.k_cache), torch.empty_like(c.v_cache)
    k[torch.from_numpy(perm)] = c.k_cache
    v[torch.from_numpy(perm)] = c.v_cache
    c.k_cache, c.v_cache = k, v
    c.block_table = torch.from_numpy(perm[c.block_table.numpy()].astype(np.int32))
    b = _run(pi)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_more_queries_than_tokens_is_refused():
    pi = make_prefill_inputs([0], [10], 8, 1, "bf16", seed=7)
    pi.cache.seq_lens[0] = 5
    with pytest.raises(ValueError):
        _run(pi)
