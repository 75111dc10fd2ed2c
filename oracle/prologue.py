"""The decode step's prologue, float64: QK-norm, RoPE and the paged KV-cache
append of the new token (with FP8 quantisation of the new K/V and,
optionally, of the query).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed.  The HPC-Ops blog (§Attention Backend: Dynamic
Load-Balanced Scheduling, the paragraph on the fused attention prologue)
names four operations fused before attention: QK-Norm, RoPE, the KV-cache
write and, in FP8, query quantisation; the German retelling (§Warum ist
dynamisches Scheduling entscheidend für Attention?) names RoPE, QK-norm and
the KV write.  Neither page gives a formula.  The plain readings used here:

* one new token per sequence b, at position p_b = the number of tokens
  already cached for b; after the step the sequence holds p_b + 1 tokens;
* QK-norm (applied first, in the blog's order): RMS normalisation of each
  head's 128 values with a learned per-dimension weight shared by all heads
  (one for queries, one for keys),
      y = x / sqrt(mean(x^2) + eps) * w;
* RoPE (applied to the normalised q and k): rotate-half form over the whole
  head, pairing dimension i with i + 64 (i < 64), angle a_i = p_b * theta^(-i/64):
      y_i      = x_i cos a_i - x_{i+64} sin a_i
      y_{i+64} = x_{i+64} cos a_i + x_i sin a_i;
* KV write: the rotated k and the unchanged v of KV head h go to row
  p_b % 64 of page block_table[b, p_b // 64], head h, of the caches;
* storage: bf16 caches round to nearest-even; an fp8 (OCP E4M3FN) cache
  stores code = e4m3(x / scale), nearest-even, saturated to +-448, with the
  cache's per-tensor scale (k_scale for K, v_scale for V); the query is
  returned in bf16 and, when asked for, as e4m3(q / q_scale);
* a sequence whose position is negative (a padding slot), lies beyond its
  block-table row or maps to a page outside the cache writes nothing to the
  cache, and its query rows are returned as zeros.

Precision of the stored codes.  Everything here is float64, rounded once at
the end to the stored format.  The one exception is the fp8 V code: V
reaches the cache through no arithmetic but the division by v_scale, so that
division is done in float32, the precision the GPU path divides in, before
rounding to E4M3 (a quantised code is decided by both sides in the same
precision).

Pinned by ``tests/test_oracle_prologue.py``: torch's rms_norm and a RoPE
written as complex multiplication, position 0 and quarter-turn closed forms,
norm preservation and composition of rotations, a hand-solved RMS case, the
cache written at exactly one slot per (sequence, KV head), and the prologue
followed by decode attention equal to attention over the appended tokens.
"""

from __future__ import annotations

import numpy as np

from .formats import (bf16_bits_to_f64, cache_bits_to_f64, f64_to_bf16_bits, f64_to_e4m3fn_bits)

PAGE = 64
HEAD_DIM = 128


def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * weight over the last axis (float64)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(weight, dtype=np.float64)


def rope_angles(position: int, theta: float, head_dim: int = HEAD_DIM) -> np.ndarray:
    """a_i = position * theta^(-2i/head_dim), i < head_dim / 2 (float64)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return float(position) * np.power(float(theta), -2.0 * i / head_dim)


def rope_rotate(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE of x [..., D] by angles [D/2] (float64)."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    c, s = np.cos(angles), np.sin(angles)
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def encode(x: np.ndarray, fmt: str, scale: float = 1.0) -> np.ndarray:
    """Stored codes of float64 values: bf16 bits, or e4m3 codes of x / scale."""
    if fmt == "bf16":
        return f64_to_bf16_bits(x)
    if fmt == "fp8_e4m3":
        return f64_to_e4m3fn_bits(np.asarray(x, dtype=np.float64) / scale)
    raise ValueError(f"unknown format {fmt!r}")


def decode_prologue(q_bits, k_bits, v_bits, q_norm_w_bits, k_norm_w_bits, positions, block_table,
                    k_cache_bits, v_cache_bits, *, kv_format: str, eps: float, theta: float,
                    k_scale: float = 1.0, v_scale: float = 1.0, q_scale: float | None = None):
    """One prologue step.

    q_bits [B][Hq][128], k_bits / v_bits [B][H_kv][128]: bf16 codes of the
    new token's projections; q_norm_w_bits / k_norm_w_bits [128]: bf16 codes;
    positions [B]; block_table [B][max_pages]; k_cache_bits / v_cache_bits
    [num_pages][H_kv][64][128] codes (uint16 bf16 or uint8 e4m3), not modified.

    Returns (q_out float64 [B][Hq][128] before rounding, q_out bf16 codes,
    q fp8 codes or None, new K cache codes, new V cache codes, k_rot float64
    [B][H_kv][128] before storage, written [B] bool).
    """
    q = bf16_bits_to_f64(q_bits)
    k = bf16_bits_to_f64(k_bits)
    v = bf16_bits_to_f64(v_bits)
    wq = bf16_bits_to_f64(q_norm_w_bits)
    wk = bf16_bits_to_f64(k_norm_w_bits)
    B, Hq, D = q.shape
    H_kv = k.shape[1]
    num_pages, max_pages = k_cache_bits.shape[0], block_table.shape[1]
    k_cache = np.array(k_cache_bits, copy=True)
    v_cache = np.array(v_cache_bits, copy=True)
    q_out = np.zeros_like(q)
    k_rot = np.zeros_like(k)
    written = np.zeros(B, dtype=bool)
    for b in range(B):
        p = int(positions[b])
        if p < 0 or p >= max_pages * PAGE:
            continue
        page = int(block_table[b, p // PAGE])
        if page < 0 or page >= num_pages:
            continue
        ang = rope_angles(p, theta, D)
        q_out[b] = rope_rotate(rms_norm(q[b], wq, eps), ang)
        k_rot[b] = rope_rotate(rms_norm(k[b], wk, eps), ang)
        row = p % PAGE
        if kv_format == "bf16":
            k_cache[page, :, row, :] = encode(k_rot[b], "bf16")
            v_cache[page, :, row, :] = v_bits[b]            # bf16 in, bf16 stored: unchanged
        else:
            k_cache[page, :, row, :] = encode(k_rot[b], "fp8_e4m3", k_scale)
            v32 = v[b].astype(np.float32) / np.float32(v_scale)     # the GPU path's division, in float32
            v_cache[page, :, row, :] = f64_to_e4m3fn_bits(v32.astype(np.float64))
        written[b] = True
    q_bf16 = encode(q_out, "bf16")
    q_fp8 = encode(q_out, "fp8_e4m3", q_scale) if q_scale is not None else None
    return q_out, q_bf16, q_fp8, k_cache, v_cache, k_rot, written


def cache_values(bits: np.ndarray, kv_format: str, scale: float = 1.0) -> np.ndarray:
    """Float64 values of stored cache codes (dequantised with `scale`)."""
    return cache_bits_to_f64(bits, kv_format) * scale
