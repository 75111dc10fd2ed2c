"""Every 64-token tile is visited exactly once: an exact count read off the
log-sum-exp.

With Q = 0 every score is exactly 0, so every valid token adds exactly
2^0 = 1 to the running sum, in fp32 without rounding (sums stay far below
2^24), and the step's log-sum-exp must be ln(L_b) for every query head of
sequence b.  A tile skipped or visited twice moves it by at least
ln(1 + 64 / L_b) (4.9e-4 at L_b = 131072, the longest sequence here), far
outside the fp32 rounding of the logarithm and of the log-sum-exp merge
(about 1e-6 at these magnitudes); a tolerance of 5e-5 separates the two.
The output is then the plain mean of each sequence's V rows, checked
against the float64 oracle like every decode result.

Covered: the device-scheduled and host-planned steps, both tile maths, bf16
and fp8 caches, the static split-KV plans, and random batches with empty
sequences and lengths at page boundaries.
"""
import math

import numpy as np
import pytest
import torch

import load_balanced_paged_step_amd as hd
from workloads import make_inputs, workload_inputs

from decode_harness import (announce, compare, run_hip, run_hip_plan, run_hip_step, run_oracle,
                            to_device)

pytestmark = pytest.mark.gpu

LSE_COUNT_TOL = 5e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hd.lib()


def _zero_q(inp):
    inp.q.zero_()
    return inp


def _check_counts(inp, got, what):
    _, lse = got
    G = inp.num_q_heads // inp.num_kv_heads
    lens = inp.seq_lens.numpy().astype(np.int64)
    for b, L in enumerate(lens):
        row = lse[b]
        if L == 0:
            assert np.all(np.isneginf(row)), f"{what}: sequence {b} is empty, lse {row}"
            continue
        err = float(np.abs(row - math.log(L)).max())
        assert err <= LSE_COUNT_TOL, (f"{what}: sequence {b} (L={L}): lse off ln(L) by {err:.2e}, "
                                      f"i.e. {np.exp(row.min()) - L:+.1f} .. {np.exp(row.max()) - L:+.1f} "
                                      f"tokens over {G * inp.num_kv_heads} heads")


def _all_paths(inp, W, what, maths=("mfma", "valu")):
    dev = to_device(inp)
    ref = run_oracle(inp)
    for m in maths:
        for name, got in (("device step", run_hip_step(inp, W, dev, tile_math=m)),
                          ("host plan", run_hip(inp, W, dev, tile_math=m))):
            tag = f"{what} {name} {m}"
            _check_counts(inp, got, tag)
            compare(inp, got, ref, tag)


@pytest.mark.parametrize("W", [256, 1024, 333, 7])
def test_skewed_batch(W):
    announce(f"tile visits, skewed 1x128K+31x4K, W={W}")
    _all_paths(_zero_q(workload_inputs(4, poison=True)), W, f"skewed W={W}")


def test_fp8_full_heads():
    announce("tile visits, fp8 64q/8kv log-uniform, W=256")
    _all_paths(_zero_q(workload_inputs(5, poison=True)), 256, "fp8 W=256", maths=("mfma",))


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_small_workloads(cfg):
    announce(f"tile visits, workload {cfg}, W=256")
    _all_paths(_zero_q(workload_inputs(cfg, poison=True)), 256, f"workload {cfg}")


@pytest.mark.parametrize("S", [1, 8, 128])
def test_static_plans(S):
    announce(f"tile visits, skewed batch, static split S={S}")
    inp = _zero_q(workload_inputs(4, poison=True))
    plan = hd.hpc_decode_plan_static(inp.seq_lens.numpy(), inp.num_kv_heads, S)
    got = run_hip_plan(inp, plan)
    _check_counts(inp, got, f"static S={S}")
    compare(inp, got, run_oracle(inp), f"static S={S}")


@pytest.mark.parametrize("seed", range(6))
def test_random_batches(seed):
    rng = np.random.default_rng(7000 + seed)
    B = int(rng.integers(1, 65))
    hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 3, 8, 16]))
    kind = rng.random(B)
    lens = np.where(kind < 0.15, 0,
                    np.where(kind < 0.35, rng.choice([1, 63, 64, 65, 127, 128, 129, 4096], B),
                             rng.integers(1, 20000, B))).astype(int)
    if B * hkv * 64 > 6000:
        lens = np.minimum(lens, 3000)
    W = int(rng.choice([1, 17, 256, 600]))
    kv = "fp8_e4m3" if rng.random() < 0.4 else "bf16"
    announce(f"tile visits, random seed={seed} B={B} G={G} hkv={hkv} W={W} {kv}")
    inp = _zero_q(make_inputs([int(x) for x in lens], G * hkv, hkv, kv, seed=8000 + seed, poison=True))
    _all_paths(inp, W, f"random seed={seed}", maths=("mfma", "valu") if G <= hd.VALU_MAX_GROUP else ("mfma",))
