"""Pins for oracle.prologue (QK-norm, RoPE, paged KV append, fp8 codes).

None of these re-types the oracle's formulas: RMS normalisation is checked
against torch's own rms_norm, RoPE against a rotation written as complex
multiplication, both against hand-solved and closed-form cases (position 0,
quarter turns, norm preservation, composition of rotations), the cache write
against the exact slot it must touch, the stored V codes against torch's
float8 cast, and the whole prologue followed by decode attention against
attention over the tokens it appended.
"""
import math

import numpy as np
import pytest
import torch

from oracle.attention import decode_attention
from oracle.formats import bf16_bits_to_f64, e4m3fn_bits_to_f64, f64_to_bf16_bits
from oracle.prologue import decode_prologue, rms_norm, rope_angles, rope_rotate
from workloads import make_prologue_inputs

D = 128


def _run(pi, kv=None):
    c = pi.cache
    return decode_prologue(pi.bits(pi.q_in), pi.bits(pi.k_in), pi.bits(pi.v_in), pi.bits(pi.q_norm_w),
                           pi.bits(pi.k_norm_w), pi.positions.numpy(), c.block_table.numpy(), c.k_bits(),
                           c.v_bits(), kv_format=c.kv_dtype, eps=pi.eps, theta=pi.theta, k_scale=c.k_scale,
                           v_scale=c.v_scale, q_scale=pi.q_scale)


# ---- RMS normalisation -------------------------------------------------------

def test_rms_norm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 7, D)) * 3.0
    w = rng.standard_normal(D)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (D,), torch.from_numpy(w), eps=1e-6).numpy()
    np.testing.assert_allclose(rms_norm(x, w, 1e-6), ref, rtol=1e-13, atol=1e-14)


def test_rms_norm_hand_solved():
    x = np.zeros(D)
    x[0], x[1] = 3.0, 4.0            # mean square 25/128
    y = rms_norm(x, np.ones(D), 0.0)
    assert math.isclose(y[0], 3.0 * math.sqrt(128) / 5.0, rel_tol=1e-15)
    assert math.isclose(y[1], 4.0 * math.sqrt(128) / 5.0, rel_tol=1e-15)
    assert np.all(y[2:] == 0)


def test_rms_norm_unit_rms_and_scale_free():
    x = np.random.default_rng(1).standard_normal((3, D))
    y = rms_norm(x, np.ones(D), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(rms_norm(37.5 * x, np.ones(D), 0.0), y, rtol=1e-14)


# ---- RoPE --------------------------------------------------------------------

def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, D))
    ang = rng.uniform(-50, 50, D // 2)
    z = (x[:, :64] + 1j * x[:, 64:]) * np.exp(1j * ang)
    y = rope_rotate(x, ang)
    np.testing.assert_allclose(y[:, :64], z.real, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(y[:, 64:], z.imag, rtol=1e-13, atol=1e-13)


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(3).standard_normal((2, D))
    ang = rope_angles(0, 10000.0)
    assert np.all(ang == 0) and np.array_equal(rope_rotate(x, ang), x)


def test_rope_quarter_turn_swaps_halves():
    x = np.random.default_rng(4).standard_normal(D)
    y = rope_rotate(x, np.full(64, math.pi / 2))
    np.testing.assert_allclose(y[:64], -x[64:], atol=1e-15)
    np.testing.assert_allclose(y[64:], x[:64], atol=1e-15)


def test_rope_preserves_norm_and_composes():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(D)
    a, b = rope_angles(1234, 10000.0), rope_angles(98765, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(rope_rotate(x, a)), np.linalg.norm(x), rtol=1e-14)
    np.testing.assert_allclose(rope_rotate(rope_rotate(x, a), b), rope_rotate(x, a + b), rtol=1e-9, atol=1e-11)
    # angles are linear in the position
    np.testing.assert_allclose(rope_angles(1234 + 98765, 10000.0), a + b, rtol=1e-15)


def test_rope_angles_hand_solved():
    a = rope_angles(1000, 10000.0)
    assert a[0] == 1000.0                                  # theta^0
    assert math.isclose(a[32], 1000.0 / 100.0, rel_tol=1e-15)   # theta^(-64/128) = 1/100
    assert math.isclose(a[16], 1000.0 / 10.0, rel_tol=1e-15)    # theta^(-32/128) = 1/10


# ---- the cache write -----------------------------------------------------------

@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_writes_exactly_one_slot_per_sequence_and_head(kv):
    pi = make_prologue_inputs([0, 63, 64, 130, 1000], 16, 2, kv, seed=6)
    q_out, q_bf16, q_fp8, kc, vc, k_rot, written = _run(pi)
    c = pi.cache
    k0, v0 = c.k_bits(), c.v_bits()
    assert written.all()
    touched = np.zeros(k0.shape[:3], dtype=bool)          # [page, head, row]
    for b, p in enumerate(pi.positions.numpy()):
        touched[c.block_table[b, p // 64], :, p % 64] = True
    assert np.array_equal(kc[~touched], k0[~touched]) and np.array_equal(vc[~touched], v0[~touched])
    for b, p in enumerate(pi.positions.numpy()):
        page, row = int(c.block_table[b, p // 64]), int(p) % 64
        if kv == "bf16":
            assert np.array_equal(vc[page, :, row], pi.bits(pi.v_in)[b])    # V stored unchanged
            assert np.array_equal(kc[page, :, row], f64_to_bf16_bits(k_rot[b]))
        else:
            # V codes: torch's float8 cast of the float32 quotient (a single rounding)
            v32 = pi.v_in[b].float() / torch.tensor(c.v_scale, dtype=torch.float32)
            ref = v32.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(vc[page, :, row], ref)
            kval = e4m3fn_bits_to_f64(kc[page, :, row]) * c.k_scale
            np.testing.assert_allclose(kval, np.clip(k_rot[b], -448 * c.k_scale, 448 * c.k_scale),
                                       rtol=2.0 ** -4, atol=2.0 ** -10 * c.k_scale)


def test_padding_and_out_of_range_positions_write_nothing():
    pi = make_prologue_inputs([100, -1, 300], 8, 1, "bf16", seed=7)
    # sequence 2: point its page at one outside the cache
    pi.cache.block_table[2, 300 // 64] = pi.cache.num_pages + 5
    q_out, q_bf16, _, kc, vc, _, written = _run(pi)
    assert written.tolist() == [True, False, False]
    assert np.all(q_out[1:] == 0) and np.all(q_bf16[1:] == 0)
    c = pi.cache
    changed = np.argwhere(np.any(kc != c.k_bits(), axis=-1))
    assert {tuple(x) for x in changed.tolist()} <= {(int(c.block_table[0, 1]), 0, 100 % 64)}


def test_query_codes():
    pi = make_prologue_inputs([5, 77], 8, 1, "bf16", seed=8)
    q_out, q_bf16, q_fp8, *_ = _run(pi)
    np.testing.assert_allclose(bf16_bits_to_f64(q_bf16), q_out, rtol=2.0 ** -8)
    ref = torch.from_numpy(q_out / pi.q_scale).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    # torch casts float64 through float32; the two agree unless float32 lands on a midpoint
    agree = np.mean(q_fp8 == ref.numpy())
    assert agree > 0.999
    np.testing.assert_allclose(e4m3fn_bits_to_f64(q_fp8) * pi.q_scale, np.clip(q_out, -448 * pi.q_scale,
                                                                               448 * pi.q_scale),
                               rtol=2.0 ** -4, atol=2.0 ** -10 * pi.q_scale)


# ---- prologue, then decode attention -------------------------------------------

@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_append_then_attend_equals_attention_over_appended_tokens(kv):
    """Fill a sequence token by token through the prologue, then decode: the
    result equals softmax attention of the last rotated query over every
    appended (stored) key and value, gathered here in position order."""
    n, Hq, Hkv = 150, 8, 2
    pi = make_prologue_inputs([n - 1], Hq, Hkv, kv, seed=9)
    c = pi.cache
    kc, vc = c.k_bits().copy(), c.v_bits().copy()
    rng = np.random.default_rng(10)
    keys, vals = [], []
    for p in range(n):
        qb = f64_to_bf16_bits(rng.standard_normal((1, Hq, D)))
        kb = f64_to_bf16_bits(rng.standard_normal((1, Hkv, D)))
        vb = f64_to_bf16_bits(rng.standard_normal((1, Hkv, D)))
        q_out, q_bf16, _, kc, vc, _, written = decode_prologue(
            qb, kb, vb, pi.bits(pi.q_norm_w), pi.bits(pi.k_norm_w), np.array([p]), c.block_table.numpy(), kc, vc,
            kv_format=kv, eps=pi.eps, theta=pi.theta, k_scale=c.k_scale, v_scale=c.v_scale)
        assert written[0]
        page, row = int(c.block_table[0, p // 64]), p % 64
        scale_k = c.k_scale if kv == "fp8_e4m3" else 1.0
        scale_v = c.v_scale if kv == "fp8_e4m3" else 1.0
        dec = e4m3fn_bits_to_f64 if kv == "fp8_e4m3" else bf16_bits_to_f64
        keys.append(dec(kc[page, :, row]) * scale_k)
        vals.append(dec(vc[page, :, row]) * scale_v)
    out, lse = decode_attention(q_bf16, kc, vc, c.block_table.numpy(), np.array([n]), num_q_heads=Hq,
                                num_kv_heads=Hkv, kv_format=kv, sm_scale=1 / math.sqrt(D), k_scale=c.k_scale,
                                v_scale=c.v_scale)
    K, V = np.stack(keys, axis=1), np.stack(vals, axis=1)          # [H_kv, n, D]
    q = bf16_bits_to_f64(q_bf16)[0]
    G = Hq // Hkv
    for hq in range(Hq):
        s = K[hq // G] @ q[hq] / math.sqrt(D)
        w = np.exp(s - s.max())
        np.testing.assert_allclose(out[0, hq], w @ V[hq // G] / w.sum(), rtol=1e-11, atol=1e-12)
        assert math.isclose(lse[0, hq], s.max() + math.log(w.sum()), rel_tol=1e-12)


def test_prologue_composition_from_independent_parts():
    """q_out and k_rot equal torch's rms_norm (with the right weight) followed
    by a complex rotation at the new token's position, for every sequence."""
    pi = make_prologue_inputs([0, 1, 4095, 131071], 16, 2, "bf16", seed=11, in_scale=4.0)
    q_out, _, _, _, _, k_rot, _ = _run(pi)
    for b, p in enumerate(pi.positions.numpy()):
        z = np.exp(1j * float(p) * 10000.0 ** (-np.arange(64) / 64.0))
        for x, w, got in ((pi.q_in[b], pi.q_norm_w, q_out[b]), (pi.k_in[b], pi.k_norm_w, k_rot[b])):
            n = torch.nn.functional.rms_norm(x.double(), (D,), w.double(), eps=pi.eps).numpy()
            r = (n[:, :64] + 1j * n[:, 64:]) * z
            np.testing.assert_allclose(got, np.concatenate([r.real, r.imag], axis=-1), rtol=1e-9, atol=1e-9)
