"""Paged GQA decode attention, float64, as its plain definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed.  The HPC-Ops blog (§Attention Backend: Dynamic
Load-Balanced Scheduling) describes decode attention over a paged KV cache
whose sequences are cut into 64-token tiles; the German retelling
(§Zwei neue HPC-Backends im vLLM-Ökosystem) gives the head shape: 64 query
heads share 8 KV heads, head dim 128.  Neither page prints the formula; the
plain reading, used here, is one query token per sequence attending to all
of that sequence's cached tokens:

    for sequence b, query head hq, KV head h = hq // G   (G = Hq / H_kv)
    k_t = k_scale * K[block_table[b, t // 64], h, t % 64, :]   t in [0, L_b)
    v_t = v_scale * V[block_table[b, t // 64], h, t % 64, :]
    s_t = sm_scale * <q[b, hq], k_t>
    out = sum_t exp(s_t - m) v_t / sum_t exp(s_t - m),   m = max_t s_t
    lse = m + ln sum_t exp(s_t - m)                       (natural log)

An empty sequence (L_b = 0) gives out = 0 and lse = -inf.

The merge of partial results (O2) is not described on the pages; the split
of one sequence's tiles over several workers in §Attention Backend implies
one.  The log-sum-exp merge is used: for parts i with (o_i, lse_i),
    M = max_i lse_i,  w_i = exp(lse_i - M),
    out = sum_i w_i o_i / sum_i w_i,  lse = M + ln sum_i w_i.

Pinned by ``tests/test_oracle_attention.py``: dense brute force through
torch's float64 scaled_dot_product_attention, closed forms (one token,
identical keys, constant values, a dominant "needle" key, a hand-solved
two-token case), page-permutation invariance and split invariance.
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, cache_bits_to_f64

PAGE = 64


def _gather_unit(k_bits, v_bits, block_table, b, h, t_lo, t_hi, kv_format, k_scale, v_scale):
    """K and V rows of tokens [t_lo, t_hi) of sequence b, KV head h, as float64."""
    t = np.arange(t_lo, t_hi, dtype=np.int64)
    pages = np.asarray(block_table)[b, t // PAGE].astype(np.int64)
    rows = t % PAGE
    K = cache_bits_to_f64(k_bits[pages, h, rows, :], kv_format) * k_scale
    V = cache_bits_to_f64(v_bits[pages, h, rows, :], kv_format) * v_scale
    return K, V


def range_attention(q_bits, k_bits, v_bits, block_table, b, h, t_lo, t_hi, *, num_q_heads,
                    num_kv_heads, kv_format="bf16", sm_scale, k_scale=1.0, v_scale=1.0):
    """(o [G, D], lse [G]) of the G query heads of KV head h over tokens [t_lo, t_hi)."""
    G = num_q_heads // num_kv_heads
    Qg = bf16_bits_to_f64(np.asarray(q_bits)[b, h * G:(h + 1) * G, :])        # [G, D]
    D = Qg.shape[1]
    if t_hi <= t_lo:
        return np.zeros((G, D)), np.full(G, -np.inf)
    K, V = _gather_unit(k_bits, v_bits, block_table, b, h, t_lo, t_hi, kv_format, k_scale, v_scale)
    S = sm_scale * (Qg @ K.T)                                                   # [G, n]
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    o = (E @ V) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def merge_partials(parts):
    """Log-sum-exp merge of [(o_i [G, D], lse_i [G])] -> (o [G, D], lse [G])."""
    os_ = np.stack([p[0] for p in parts])            # [n, G, D]
    ls = np.stack([p[1] for p in parts])             # [n, G]
    M = ls.max(axis=0)                               # [G]
    if np.all(np.isneginf(M)):
        return np.zeros(os_.shape[1:]), np.full(ls.shape[1], -np.inf)
    w = np.exp(ls - M)                               # [n, G]
    den = w.sum(axis=0)
    out = (w[:, :, None] * os_).sum(axis=0) / den[:, None]
    return out, M + np.log(den)


def decode_attention(q_bits, k_bits, v_bits, block_table, seq_lens, *, num_q_heads, num_kv_heads,
                     kv_format="bf16", sm_scale, k_scale=1.0, v_scale=1.0):
    """Full decode step: (out [B, Hq, D] float64, lse [B, Hq] float64)."""
    q_bits = np.asarray(q_bits)
    B, Hq, D = q_bits.shape
    G = num_q_heads // num_kv_heads
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        for h in range(num_kv_heads):
            o, l = range_attention(q_bits, k_bits, v_bits, block_table, b, h, 0, L,
                                   num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                                   kv_format=kv_format, sm_scale=sm_scale,
                                   k_scale=k_scale, v_scale=v_scale)
            out[b, h * G:(h + 1) * G] = o
            lse[b, h * G:(h + 1) * G] = l
    return out, lse


def split_decode_attention(q_bits, k_bits, v_bits, block_table, seq_lens, entries, *, num_q_heads,
                           num_kv_heads, kv_format="bf16", sm_scale, k_scale=1.0, v_scale=1.0):
    """Decode step computed piecewise: one (o, lse) per (unit, tile range) entry, then merged.

    ``entries`` is an iterable of (unit, t0, t1) with unit = b * H_kv + h and
    [t0, t1) a range of 64-token tiles.  Returns (out, lse, partials) where
    ``partials[i]`` is entry i's (o, lse) before the merge.
    """
    q_bits = np.asarray(q_bits)
    B, Hq, D = q_bits.shape
    G = num_q_heads // num_kv_heads
    by_unit: dict[int, list] = {}
    partials = []
    for (u, t0, t1) in entries:
        b, h = divmod(int(u), num_kv_heads)
        L = int(seq_lens[b])
        lo, hi = min(t0 * PAGE, L), min(t1 * PAGE, L)
        p = range_attention(q_bits, k_bits, v_bits, block_table, b, h, lo, hi,
                            num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                            kv_format=kv_format, sm_scale=sm_scale, k_scale=k_scale,
                            v_scale=v_scale)
        partials.append(p)
        by_unit.setdefault(int(u), []).append(p)
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for u, parts in by_unit.items():
        b, h = divmod(u, num_kv_heads)
        o, l = merge_partials(parts)
        out[b, h * G:(h + 1) * G] = o
        lse[b, h * G:(h + 1) * G] = l
    return out, lse, partials
