"""Causal prefill / extend attention over the paged KV cache, float64, as its
plain definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed.  The HPC-Ops blog (§Attention Across Prefill, Extend and
Decode Shapes) measures the same attention backend on prefill ("q512") and
extend shapes besides decode; it prints no formula.  The plain reading, used
here: sequence b holds L_b tokens in the cache, of which the last n_b are
this step's new tokens (their K/V already written, as the prologue does for
decode); each new token is a query, and query j of sequence b, at position
p = L_b - n_b + j, attends causally to the cached tokens t <= p:

    h = hq // G (G = Hq / H_kv)
    k_t = k_scale * K[block_table[b, t // 64], h, t % 64, :],  v_t likewise
    s_t = sm_scale * <q[q_start[b] + j, hq], k_t>      for t in [0, p]
    out = sum_t exp(s_t - m) v_t / sum_t exp(s_t - m),  m = max_t s_t
    lse = m + ln sum_t exp(s_t - m)

Pure prefill is n_b = L_b (the first query sees one token); decode is
n_b = 1 (the one query sees all L_b tokens).  Queries are packed: sequence
b's are rows [q_start[b], q_start[b + 1]) of q [total][Hq][128].

Pinned by ``tests/test_oracle_prefill.py``: torch's float64
scaled_dot_product_attention with is_causal (prefill) and with an explicit
mask (extend) on contiguous K/V gathered in the test, the decode oracle for
n_b = 1 and for the last query of every chunk, query 0 of a prefill
returning V_0 exactly, and page-permutation invariance.
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, cache_bits_to_f64

PAGE = 64


def prefill_attention(q_bits, k_bits, v_bits, block_table, seq_lens, q_start, *, num_q_heads: int,
                      num_kv_heads: int, kv_format: str = "bf16", sm_scale: float, k_scale: float = 1.0,
                      v_scale: float = 1.0):
    """Returns (out float64 [total][Hq][128], lse float64 [total][Hq])."""
    q = bf16_bits_to_f64(q_bits)
    total = q.shape[0]
    G = num_q_heads // num_kv_heads
    out = np.zeros((total, num_q_heads, q.shape[2]))
    lse = np.full((total, num_q_heads), -np.inf)
    block_table = np.asarray(block_table)
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        r0, r1 = int(q_start[b]), int(q_start[b + 1])
        n = r1 - r0
        if n > L:
            raise ValueError(f"sequence {b}: {n} queries but only {L} cached tokens")
        if n == 0:
            continue
        pages = block_table[b, :(L + PAGE - 1) // PAGE]
        K = cache_bits_to_f64(k_bits[pages], kv_format) * k_scale        # [pages, H_kv, 64, D]
        V = cache_bits_to_f64(v_bits[pages], kv_format) * v_scale
        K = K.transpose(1, 0, 2, 3).reshape(num_kv_heads, -1, K.shape[-1])[:, :L]   # [H_kv, L, D]
        V = V.transpose(1, 0, 2, 3).reshape(num_kv_heads, -1, V.shape[-1])[:, :L]
        pos = L - n + np.arange(n)                                        # each query's position
        visible = np.arange(L)[None, :] <= pos[:, None]                   # [n, L]
        for hq in range(num_q_heads):
            h = hq // G
            s = sm_scale * (q[r0:r1, hq, :] @ K[h].T)                     # [n, L]
            s = np.where(visible, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            l = e.sum(axis=1, keepdims=True)
            out[r0:r1, hq, :] = (e @ V[h]) / l
            lse[r0:r1, hq] = (m + np.log(l))[:, 0]
    return out, lse
