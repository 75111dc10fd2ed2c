"""The in-kernel merge of the device-scheduled step (fused_merge = 1): the
decode kernel's last-arriving worker of every split unit merges the unit's
partials, and no merge kernel runs.

Checked against the float64 oracle like every decode result (max|out -
oracle| <= 1e-2 max|V| for bf16 KV, 3e-2 for fp8; per (sequence, KV head)
unit max|out_u - oracle_u| <= 1e-2 max|oracle_u| + 1e-6; |lse - oracle| <=
1e-3 / 1e-2), with exact tile-visit counts (Q = 0: lse = ln L_b, as in
test_tile_visits_gpu.py), for both tile maths, and over repeated steps that
reuse one workspace while the lengths change, since each unit's arrival
count lives in the workspace and every step must leave it at zero.
"""
import math

import numpy as np
import pytest
import torch

import load_balanced_paged_step_amd as hd
from workloads import make_inputs, workload_inputs

from decode_harness import announce, compare, run_hip_step, run_oracle, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hd.lib()


def _fused(inp, W, what, dev=None, tile_math="mfma", ref=None):
    dev = dev or to_device(inp)
    ref = ref if ref is not None else run_oracle(inp)
    got = run_hip_step(inp, W, dev, tile_math=tile_math, fused_merge=True)
    compare(inp, got, ref, f"{what} fused {tile_math}")
    return got, ref


@pytest.mark.parametrize("cfg,W", [(1, 256), (1, 3), (2, 256), (3, 256), (3, 7), (4, 256), (4, 1024)])
def test_bf16_workloads(cfg, W):
    announce(f"fused merge, workload {cfg}, W={W}")
    inp = workload_inputs(cfg, poison=True)
    dev = to_device(inp)
    ref = run_oracle(inp)
    for m in ("mfma", "valu"):
        _fused(inp, W, f"workload {cfg} W={W}", dev, m, ref)


def test_fp8_full_heads():
    announce("fused merge, fp8 workload 5, W=256")
    _fused(workload_inputs(5, poison=True), 256, "workload 5")


@pytest.mark.parametrize("cfg,W", [(2, 256), (3, 256), (4, 256), (4, 333)])
def test_tile_visits_counted(cfg, W):
    announce(f"fused merge, tile visits, workload {cfg}, W={W}")
    inp = workload_inputs(cfg, poison=True)
    inp.q.zero_()
    (_, lse), _ = _fused(inp, W, f"counts workload {cfg}")
    for b, L in enumerate(inp.seq_lens.numpy()):
        if L == 0:
            assert np.all(np.isneginf(lse[b]))
        else:
            assert float(np.abs(lse[b] - math.log(int(L))).max()) <= 5e-5, (b, int(L))


@pytest.mark.parametrize("seed", range(6))
def test_random_batches(seed):
    rng = np.random.default_rng(9000 + seed)
    B = int(rng.integers(1, 81))
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 3, 8, 16]))
    kind = rng.random(B)
    lens = np.where(kind < 0.15, 0,
                    np.where(kind < 0.3, rng.choice([1, 63, 64, 65, 127, 128, 129], B),
                             rng.integers(1, 4000, B))).astype(int)
    if B * hkv * 64 > 6000:
        lens = np.minimum(lens, 600)
    W = int(rng.choice([1, 3, 17, 64, 256, 333, 600]))
    kv = "fp8_e4m3" if rng.random() < 0.4 else "bf16"
    announce(f"fused merge, random seed={seed} B={B} G={G} hkv={hkv} W={W} {kv}")
    inp = make_inputs([int(x) for x in lens], G * hkv, hkv, kv, seed=9500 + seed, poison=True)
    dev = to_device(inp)
    ref = run_oracle(inp)
    for m in (("mfma", "valu") if G <= hd.VALU_MAX_GROUP else ("mfma",)):
        _fused(inp, W, f"random seed={seed}", dev, m, ref)


@pytest.mark.parametrize("lens,hq,hkv,kv", [
    ([128] * 8, 8, 1, "bf16"),             # 16 tiles, 2 workers per sequence
    ([512] * 8, 8, 1, "bf16"),             # 64 tiles, 8: the most the merge rule keeps in the kernel
    ([512] * 2, 64, 8, "fp8_e4m3"),        # 128 tiles, 8 per (sequence, KV head)
    ([37, 80, 150, 200], 8, 1, "bf16"),    # one worker per tile
])
def test_batches_the_merge_rule_keeps_in_the_kernel(lens, hq, hkv, kv):
    """The step as the library's rules set it up (worker count, entry price,
    merge mode) on batches with no more tiles than workers and 2 to 8 workers
    per unit, for which hpc_decode_pick_merge picks the in-kernel merge."""
    W = hd.hpc_decode_pick_workers(np.array(lens), hkv, kv, 256)
    price = hd.hpc_decode_pick_entry_price(np.array(lens), hkv, kv, W)
    assert hd.hpc_decode_pick_merge(np.array(lens), hkv, W, price)
    announce(f"merge rule batch {len(lens)}x{lens[0]} {hq}q/{hkv}kv {kv} W={W} price={price}")
    inp = make_inputs(lens, hq, hkv, kv, seed=77, poison=True)
    dev = to_device(inp)
    got = run_hip_step(inp, W, dev, fused_merge=True, entry_price=price)
    compare(inp, got, run_oracle(inp), f"merge rule batch {len(lens)}x{lens[0]}")


def test_repeated_steps_reuse_the_workspace():
    """Twelve steps on one zero-filled workspace, with the lengths (and so
    every unit's number of sharing workers) changing from step to step and
    the merge mode switched back and forth: each step matches the oracle."""
    rng = np.random.default_rng(4242)
    B, hkv, G, W, max_pages = 24, 2, 8, 256, 80
    base = make_inputs([64 * max_pages] * B, G * hkv, hkv, "bf16", seed=4243, max_pages_per_seq=max_pages)
    dev = to_device(base)
    ws = torch.zeros(hd.hpc_decode_step_workspace_size(B, G * hkv, hkv, W), dtype=torch.uint8, device="cuda")
    for step in range(12):
        lens = rng.integers(0, 64 * max_pages + 1, size=B)
        lens[rng.random(B) < 0.1] = 0
        base.seq_lens = torch.from_numpy(lens.astype(np.int32))
        dev["sl"] = base.seq_lens.cuda()
        fused = step % 4 != 3
        announce(f"fused merge, repeated step {step} fused={fused} lens[:4]={lens[:4].tolist()}")
        got = run_hip_step(base, W, dev, fused_merge=fused, workspace=ws)
        compare(base, got, run_oracle(base), f"repeated step {step}")
