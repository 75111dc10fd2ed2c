"""The per-unit output bound of the GPU parity checks, exercised on the CPU.

The global bound max|out - ref| <= 1e-2 max|V| cannot see the 131072-token
sequence of the skewed batch: that sequence's whole output is below it.  The
per-unit bound (max|out_u - ref_u| <= 1e-2 max|ref_u| + 1e-6 for every
(sequence, KV head)) must reject a zeroed, a halved or a sign-flipped unit,
and must accept the oracle's result carried through the kernel's own
roundings (probabilities and output in bf16).
"""
import numpy as np
import pytest
import torch

from oracle import cache_bits_to_f64, decode_attention
from workloads import make_inputs, workload_inputs

from decode_harness import OUT_TOL, max_abs_v, unit_check


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).bfloat16().double().numpy()


def _rounded_like_kernel(inp):
    """Attention with P and the output rounded to bf16 (the kernel's two
    roundings), per unit, in float64 otherwise."""
    K = cache_bits_to_f64(inp.k_bits(), inp.kv_dtype) * inp.k_scale
    V = cache_bits_to_f64(inp.v_bits(), inp.kv_dtype) * inp.v_scale
    Q = inp.q.double().numpy()
    G = inp.num_q_heads // inp.num_kv_heads
    out = np.zeros(Q.shape)
    for b, L in enumerate(inp.seq_lens.numpy()):
        if L == 0:
            continue
        pages = inp.block_table.numpy()[b, :(L + 63) // 64]
        for h in range(inp.num_kv_heads):
            k = K[pages, h].reshape(-1, 128)[:L]
            v = V[pages, h].reshape(-1, 128)[:L]
            s = Q[b, h * G:(h + 1) * G] @ k.T * inp.sm_scale
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[b, h * G:(h + 1) * G] = _bf16((_bf16(p) @ v) / p.sum(axis=1, keepdims=True))
    return out


def _oracle(inp):
    return decode_attention(inp.q_bits(), inp.k_bits(), inp.v_bits(), inp.block_table.numpy(),
                            inp.seq_lens.numpy(), num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads,
                            kv_format=inp.kv_dtype, sm_scale=inp.sm_scale, k_scale=inp.k_scale,
                            v_scale=inp.v_scale)


def test_global_bound_is_blind_to_the_long_sequence():
    inp = workload_inputs(4)
    ref_out, _ = _oracle(inp)
    assert np.abs(ref_out[0]).max() < OUT_TOL["bf16"] * max_abs_v(inp)   # the reason for the unit bound
    bad = ref_out.copy()
    bad[0] = 0.0
    with pytest.raises(AssertionError, match=r"unit \(seq 0, kv head 0\)"):
        unit_check(bad, ref_out, inp.num_kv_heads, "zeroed 128K unit")


@pytest.mark.parametrize("fault", ["halved", "negated", "one head zeroed", "one dim off"])
def test_unit_faults_are_caught(fault):
    inp = make_inputs([5000, 300, 64, 1], 16, 2, "bf16", seed=12)
    ref_out, _ = _oracle(inp)
    bad = ref_out.copy()
    if fault == "halved":
        bad[1, 8:16] *= 0.5
    elif fault == "negated":
        bad[0, 0:8] *= -1.0
    elif fault == "one head zeroed":
        bad[0, 3] = 0.0
    else:
        d = int(np.argmax(np.abs(ref_out[2, 9])))
        bad[2, 9, d] *= 1.05
    with pytest.raises(AssertionError, match="unit"):
        unit_check(bad, ref_out, inp.num_kv_heads, fault)


@pytest.mark.parametrize("cfg", [1, 4])
def test_kernel_roundings_pass(cfg):
    inp = workload_inputs(cfg)
    ref_out, _ = _oracle(inp)
    ratio, _ = unit_check(_rounded_like_kernel(inp), ref_out, inp.num_kv_heads, f"workload {cfg}")
    assert 0 < ratio < 5e-3


def test_fp8_kernel_roundings_pass():
    inp = make_inputs([20000, 129, 3000, 0], 32, 4, "fp8_e4m3", seed=5)
    ref_out, _ = _oracle(inp)
    ratio, _ = unit_check(_rounded_like_kernel(inp), ref_out, inp.num_kv_heads, "fp8")
    assert 0 < ratio < 5e-3
