"""Parity of the VALU tile math (tile_math = HPC_TILE_MATH_VALU: bf16 dot2
products on the vector ALU, no MFMA) against the float64 oracle, through the
C ABI, with the host-planned and the device-scheduled step.

The VALU path computes the same attention as the MFMA one: scores from bf16
K and Q with fp32 accumulation, an exp2-domain online softmax, P rounded to
bf16 for P V with fp32 accumulation.  Tolerances are the same as for every
decode result: max|out - oracle| <= 1e-2 max|V| (bf16 KV) or 3e-2 max|V|
(fp8 KV, oracle on the dequantised cache); per (sequence, KV head) unit
max|out_u - oracle_u| <= 1e-2 max|oracle_u| + 1e-6; |lse - oracle| <= 1e-3
(bf16) or 1e-2 (fp8).
"""
import numpy as np
import pytest
import torch

import load_balanced_paged_step_amd as hd
from workloads import make_inputs, workload_inputs

from decode_harness import announce, compare, run_hip, run_hip_step, run_oracle, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hd.lib()


def _both(inp, W, what, dev=None):
    """VALU host-planned and device-scheduled steps, each against the oracle."""
    dev = dev or to_device(inp)
    ref = run_oracle(inp)
    a = run_hip(inp, W, dev, tile_math="valu")
    b = run_hip_step(inp, W, dev, tile_math="valu")
    compare(inp, a, ref, f"{what} valu host plan")
    compare(inp, b, ref, f"{what} valu device step")
    return a, b, ref


@pytest.mark.parametrize("W", [1, 2, 3, 7, 256, 1024])
def test_tiny_workload(W):
    announce(f"valu tiny workload, poisoned, W={W}")
    _both(workload_inputs(1, poison=True), W, f"tiny W={W}")


@pytest.mark.parametrize("cfg,W", [(2, 256), (3, 256), (3, 7), (4, 256), (4, 1024)])
def test_bf16_workloads(cfg, W):
    announce(f"valu workload {cfg}, poisoned, W={W}")
    _both(workload_inputs(cfg, poison=True), W, f"workload {cfg} W={W}")


def test_fp8_full_head_workload():
    announce("valu fp8 workload 5, W=256")
    _both(workload_inputs(5, poison=True), 256, "workload 5 W=256")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("G", [1, 2, 3, 5, 7, 8])
def test_group_sizes(G, kv):
    """Every group size the VALU path holds (heads beyond G are computed on
    zero Q rows and never written), ragged and empty sequences, two KV heads."""
    announce(f"valu group size G={G} {kv}")
    inp = make_inputs([700, 0, 65, 3000, 1], 2 * G, 2, kv, seed=300 + G, poison=True)
    _both(inp, 13, f"G={G} {kv}")


@pytest.mark.parametrize("seed", range(8))
def test_random_batches(seed):
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 81))
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.integers(1, 9))
    kind = rng.random(B)
    lens = np.where(kind < 0.15, 0,
                    np.where(kind < 0.3, rng.choice([1, 63, 64, 65, 127, 128, 129], B),
                             rng.integers(1, 4000, B))).astype(int)
    if B * hkv * 64 > 6000:
        lens = np.minimum(lens, 600)
    W = int(rng.choice([1, 3, 17, 64, 256, 333, 600]))
    kv = "fp8_e4m3" if rng.random() < 0.4 else "bf16"
    announce(f"valu random batch seed={seed} B={B} G={G} hkv={hkv} W={W} {kv}")
    inp = make_inputs([int(x) for x in lens], G * hkv, hkv, kv, seed=6000 + seed, poison=True)
    _both(inp, W, f"random seed={seed}")


def _plant_rising_scores(inp, b, h_kv, scale):
    """Make sequence b's keys line up more and more with query head
    h_kv*G's direction as the token index grows, so the running max of every
    tile exceeds the last one (each tile must rescale the running sums)."""
    G = inp.num_q_heads // inp.num_kv_heads
    q = inp.q[b, h_kv * G].float()
    L = int(inp.seq_lens[b])
    for t in range(L):
        page = int(inp.block_table[b, t // 64])
        row = inp.k_cache[page, h_kv, t % 64].float()
        inp.k_cache[page, h_kv, t % 64] = (row * 0.1 + q * (scale * t / L)).to(inp.k_cache.dtype)


def test_running_max_grows_every_tile():
    announce("valu rising scores (a rescale in every tile)")
    inp = make_inputs([1000, 333, 64], 8, 1, "bf16", seed=77)
    for b in range(3):
        _plant_rising_scores(inp, b, 0, 0.25)
    for W in (1, 5, 256):
        _both(inp, W, f"rising W={W}")


def test_needle_key():
    """One key far above the others in the middle of a long sequence: the
    output of its head is that token's value row."""
    announce("valu needle key")
    inp = make_inputs([5000], 8, 1, "bf16", seed=91)
    t = 2777
    page = int(inp.block_table[0, t // 64])
    q0 = inp.q[0, 0].float()
    inp.k_cache[page, 0, t % 64] = (q0 * 4.0).to(torch.bfloat16)
    a, b, ref = _both(inp, 256, "needle")
    v = inp.v_cache[page, 0, t % 64].double().numpy()
    assert np.abs(ref[0][0, 0] - v).max() < 1e-2
    assert np.abs(a[0][0, 0] - v).max() < 2e-2 and np.abs(b[0][0, 0] - v).max() < 2e-2


def test_bitwise_deterministic():
    inp = workload_inputs(4)
    dev = to_device(inp)
    announce("valu determinism, workload 4")
    r1 = run_hip_step(inp, 256, dev, tile_math="valu")
    r2 = run_hip_step(inp, 256, dev, tile_math="valu")
    assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])


def test_device_schedule_size_limit():
    """2048 sequences (the device schedule's largest batch), where the LDS of
    the VALU instantiation is fullest (its two pending entry slots plus the
    lengths and their prefix)."""
    rng = np.random.default_rng(2048)
    lens = rng.integers(0, 300, size=2048)
    lens[rng.random(2048) < 0.1] = 0
    announce("valu device step at 2048 sequences, 2 kv heads")
    inp = make_inputs([int(x) for x in lens], 8, 2, "bf16", seed=7, poison=True)
    compare(inp, run_hip_step(inp, 256, tile_math="valu"), run_oracle(inp), "valu 2048 sequences")


def test_group_above_eight_is_refused():
    inp = make_inputs([100, 200], 16, 1, "bf16", seed=3)
    dev = to_device(inp)
    with pytest.raises(hd.HpcDecodeError):
        run_hip_step(inp, 8, dev, tile_math="valu")
