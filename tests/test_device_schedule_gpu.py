"""The schedule derived on the GPU (hpc_decode_plan_device / hpc_decode_step)
against the host planner and the oracle.

* plan words materialised on the device equal the oracle's schedule word for
  word (every tile covered once, same entries, slots and merge records);
* a device-scheduled step matches the host-planned step: bitwise for every
  sequence that one worker finishes alone (same schedule, same arithmetic),
  and to fp32 rounding for split sequences, whose partials the merge kernel
  may fold in another order (its grid, and so the lanes that take each
  partial, is sized from the number of merge records, which differs between
  the two schedules); both match the float64 oracle;
* both hold at the device schedule's limits (2048 sequences, 4096 units,
  65536 workers).
"""
import numpy as np
import pytest
import torch

import load_balanced_paged_step_amd as hd
from oracle import build_plan
from workloads import make_inputs, workload_inputs

from decode_harness import announce, compare, run_hip, run_hip_plan, run_hip_step, run_oracle, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hd.lib()


def _device_plan(lens, H, W, max_pages=None, entry_price=0):
    lens = np.asarray(lens, dtype=np.int32)
    mp = max_pages or max(1, int((lens.max() + 63) // 64) if lens.size else 1)
    sl = torch.from_numpy(lens).cuda()
    plan = hd.hpc_decode_plan_device(sl, H, W, mp, entry_price=entry_price)
    torch.cuda.synchronize()
    words = plan.cpu().numpy()
    return words[:hd.hpc_decode_plan_words(words)]


@pytest.mark.parametrize("lens,H,W", [
    ([37, 64, 130, 200], 1, 4), ([0, 100, 10], 2, 4), ([65], 1, 5), ([1, 0, 128], 1, 1),
    ([131072] + [4096] * 31, 1, 256), ([131072] + [4096] * 31, 1, 1024), ([512] * 64, 1, 256),
    ([1024] * 8, 1, 256), ([0, 0, 0], 8, 7), ([5000] * 3, 8, 700), ([1] * 300, 2, 37),
])
def test_device_plan_equals_oracle(lens, H, W):
    announce(f"device plan lens[:4]={lens[:4]} B={len(lens)} H={H} W={W}")
    assert np.array_equal(_device_plan(lens, H, W), build_plan(lens, H, W))


@pytest.mark.parametrize("lens,H,W", [
    ([2 ** 28 - 1, 5, 2 ** 27 + 13, 0] * 4, 8, 2047),     # T near 2^29 tiles: large w T / W quotients
    ([2 ** 28] * 16, 8, 2048),
    ([64 * 2047 - 1, 1, 1, 1], 1, 2048),                     # W just above T
    ([100] * 5, 3, 2048),                                    # W far above T: one tile per worker
    ([64 * 4096 + 1] * 3, 2, 1999),
])
def test_device_plan_extreme_quotients(lens, H, W):
    announce(f"device plan extreme B={len(lens)} H={H} W={W}")
    assert np.array_equal(_device_plan(lens, H, W), build_plan(lens, H, W))


def test_device_plan_random_batches():
    rng = np.random.default_rng(123)
    for i in range(60):
        B = int(rng.integers(1, 64))
        H = int(rng.integers(1, 9))
        W = int(rng.integers(1, 1500))
        lens = rng.integers(0, 20000, size=B)
        lens[rng.random(B) < 0.2] = 0
        announce(f"device plan random #{i} B={B} H={H} W={W}")
        assert np.array_equal(_device_plan(lens, H, W), build_plan(lens, H, W)), (lens.tolist(), H, W)


def test_device_plan_of_fp8_workload():
    inp = workload_inputs(5)
    lens = inp.seq_lens.numpy()
    for W in (256, 1024):
        announce(f"device plan workload 5 W={W}")
        assert np.array_equal(_device_plan(lens, 8, W), build_plan(lens, 8, W))


def assert_same_as_host_planned(inp, W, a, b, plan=None):
    if plan is None:
        plan = build_plan(inp.seq_lens.numpy(), inp.num_kv_heads, W)
    hdr_W, E = int(plan[3]), int(plan[5])
    ents = plan[16 + hdr_W + 1:16 + hdr_W + 1 + 4 * E].reshape(E, 4)
    G = inp.num_q_heads // inp.num_kv_heads
    single = np.zeros(inp.batch * inp.num_kv_heads, dtype=bool)
    single[ents[ents[:, 3] < 0, 0]] = True
    rows = np.repeat(single, G).reshape(inp.batch, inp.num_q_heads)
    assert np.array_equal(a[0][rows], b[0][rows]) and np.array_equal(a[1][rows], b[1][rows])
    np.testing.assert_allclose(a[0], b[0], rtol=2.0 ** -7, atol=1e-6)
    fin = np.isfinite(b[1])
    assert np.array_equal(fin, np.isfinite(a[1]))
    np.testing.assert_allclose(a[1][fin], b[1][fin], rtol=0, atol=4e-6)


def run_step(inp, W, dev=None, entry_price=0):
    if dev is None:
        dev = to_device(inp)
    out = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    launch = hd.StepLauncher(dev["q"], dev["k"], dev["v"], dev["bt"], dev["sl"], out, lse,
                             num_kv_heads=inp.num_kv_heads, n_workers=W, sm_scale=inp.sm_scale,
                             k_scale=inp.k_scale, v_scale=inp.v_scale, entry_price=entry_price)
    launch()
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("cfg,W", [(1, 3), (1, 256), (2, 256), (3, 256), (4, 256), (4, 1024), (5, 256), (4, 252), (5, 255), (5, 512)])
def test_step_equals_host_planned(cfg, W):
    inp = workload_inputs(cfg, poison=True)
    dev = to_device(inp)
    announce(f"device step vs host plan, workload {cfg}, W={W}")
    a = run_step(inp, W, dev)
    b = run_hip(inp, W, dev)
    assert_same_as_host_planned(inp, W, a, b)
    compare(inp, a, run_oracle(inp), f"device step workload {cfg} W={W}")


@pytest.mark.parametrize("lens,hq,hkv,W", [
    ([0, 0, 0], 8, 1, 4), ([0, 37, 0, 1], 8, 1, 3), ([1] * 9, 8, 1, 4),
    ([63, 64, 65, 127, 128, 129], 8, 1, 5), ([500, 30], 16, 1, 6), ([300, 1000, 7], 12, 3, 11),
    ([4000, 17], 64, 8, 64), ([2] * 700, 8, 1, 256),
    # 64 and 65 sequences (one and two 64-lane rounds of the prefix scan), many of them empty
    ([0, 5, 0, 130] * 16, 8, 1, 40), ([0, 5, 0, 130] * 16 + [64], 8, 1, 40), ([64] * 64, 16, 2, 300),
])
def test_step_edge_shapes(lens, hq, hkv, W):
    inp = make_inputs(lens, hq, hkv, "bf16", seed=len(lens) + hq, poison=True)
    announce(f"device step edge lens[:4]={lens[:4]} B={len(lens)} hq={hq} hkv={hkv} W={W}")
    dev = to_device(inp)
    a = run_step(inp, W, dev)
    b = run_hip(inp, W, dev)
    assert_same_as_host_planned(inp, W, a, b)
    compare(inp, a, run_oracle(inp), "device step edge")


def test_step_clamps_lengths_to_the_block_table():
    """Device lengths beyond max_pages * 64 are clamped, never read past the table."""
    inp = make_inputs([100, 200], 8, 1, "bf16", seed=11, max_pages_per_seq=4)
    dev = to_device(inp)
    dev["sl"] = torch.tensor([100, 10_000], dtype=torch.int32, device="cuda")
    announce("device step with an over-long length")
    a = run_step(inp, 8, dev)
    inp.seq_lens = torch.tensor([100, 256], dtype=torch.int32)      # what the clamp leaves
    compare(inp, a, run_oracle(inp), "clamped")


def test_repeated_device_steps_with_changing_splits():
    """One workspace reused across steps whose lengths change which sequences
    are split (and which are empty): no merge record of an earlier step
    leaks into a later one."""
    base = make_inputs([7000, 300, 65, 4000], 16, 2, "bf16", seed=17, max_pages_per_seq=130)
    dev = to_device(base)
    out = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    sl = dev["sl"]
    launch = hd.StepLauncher(dev["q"], dev["k"], dev["v"], dev["bt"], sl, out, lse, num_kv_heads=2,
                             n_workers=64, sm_scale=base.sm_scale)
    for i, lens in enumerate(([7000, 300, 65, 4000], [7001, 0, 66, 4100], [8000, 1, 64, 8300],
                              [100, 200, 300, 400], [0, 0, 0, 0], [7000, 300, 65, 4000])):
        announce(f"repeated device step {i} lens={lens}")
        sl.copy_(torch.tensor(lens, dtype=torch.int32))
        launch()
        torch.cuda.synchronize()
        base.seq_lens = torch.tensor(lens, dtype=torch.int32)
        got = (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))
        compare(base, got, run_oracle(base), f"step {i}")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
@pytest.mark.parametrize("G", [1, 2, 3, 5, 7, 16])
def test_group_sizes_both_schedules(G, kv):
    """Every GQA group size up to the largest supported, ragged and empty
    sequences, two KV heads: both schedules against the oracle, and against
    each other."""
    lens = [700, 0, 65, 3000, 1]
    inp = make_inputs(lens, 2 * G, 2, kv, seed=100 + G, poison=True)
    announce(f"group size G={G} {kv}")
    dev = to_device(inp)
    a = run_step(inp, 13, dev)
    b = run_hip(inp, 13, dev)
    assert_same_as_host_planned(inp, 13, a, b)
    ref = run_oracle(inp)
    compare(inp, a, ref, f"device step G={G} {kv}")
    compare(inp, b, ref, f"host plan G={G} {kv}")


def _random_case(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 81))
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.integers(1, 17))
    kind = rng.random(B)
    lens = np.where(kind < 0.15, 0,
                    np.where(kind < 0.3, rng.choice([1, 63, 64, 65, 127, 128, 129], B),
                             rng.integers(1, 4000, B))).astype(int)
    if B * hkv * 64 > 6000:           # keep the oracle quick: shorten big batches
        lens = np.minimum(lens, 600)
    W = int(rng.choice([1, 3, 17, 64, 256, 333, 600]))
    kv = "fp8_e4m3" if rng.random() < 0.4 else "bf16"
    return [int(x) for x in lens], G * hkv, hkv, W, kv


@pytest.mark.parametrize("seed", range(12))
def test_random_batches_both_schedules(seed):
    """Seeded random batches: sizes, lengths (zeros and page-boundary values
    included), group sizes, KV head counts, worker counts and KV types."""
    lens, hq, hkv, W, kv = _random_case(1000 + seed)
    announce(f"random batch seed={seed} B={len(lens)} hq={hq} hkv={hkv} W={W} {kv} lens[:6]={lens[:6]}")
    inp = make_inputs(lens, hq, hkv, kv, seed=2000 + seed, poison=True)
    dev = to_device(inp)
    a = run_step(inp, W, dev)
    b = run_hip(inp, W, dev)
    assert_same_as_host_planned(inp, W, a, b)
    ref = run_oracle(inp)
    compare(inp, a, ref, f"random device step seed={seed}")
    compare(inp, b, ref, f"random host plan seed={seed}")


def _limit_lengths():
    rng = np.random.default_rng(2048)
    lens = rng.integers(0, 300, size=2048)
    lens[rng.random(2048) < 0.1] = 0
    return lens


def test_device_plan_at_its_limits():
    """The plan-materialising kernel at its largest batch, units and workers."""
    lens = _limit_lengths()
    announce("device plan at the limits: B=2048 H=2 W=2048")
    assert np.array_equal(_device_plan(lens, 2, 2048), build_plan(lens, 2, 2048))


@pytest.mark.parametrize("W", [4099, 65536])
def test_step_at_the_size_limits(W):
    """The device-scheduled step at its largest batch (2048 sequences, 4096
    units) and worker count (65536, far more workers than tiles) against the
    host-planned step and the oracle.  The host plan here is the C++
    planner's, which the CPU tests hold equal to the oracle's word for word
    (the oracle's planner is too slow at 65536 workers)."""
    lens = _limit_lengths()
    inp = make_inputs(lens, 8, 2, "bf16", seed=7, poison=True)
    announce(f"device step at the limits: B=2048 hq=8 hkv=2 W={W}")
    dev = to_device(inp)
    a = run_step(inp, W, dev)
    b = run_hip(inp, W, dev)
    assert_same_as_host_planned(inp, W, a, b, plan=hd.hpc_decode_plan(inp.seq_lens.numpy(), 2, W))
    compare(inp, a, run_oracle(inp), f"device step at the limits W={W}")


# ------------------------------------------------------ priced partition ---

PRICED_PLAN_CASES = [
    ([37, 64, 130, 200], 1, 4), ([0, 100, 10], 2, 4), ([64, 64, 64, 640], 1, 2), ([64, 0, 192], 2, 2),
    ([131072] + [4096] * 31, 1, 252), ([131072] + [4096] * 31, 1, 256), ([512] * 64, 1, 256),
    ([5000] * 3, 8, 700), ([1] * 300, 2, 37), ([0, 5, 0, 130] * 16 + [64], 8, 40), ([0, 0, 0], 8, 7),
]


@pytest.mark.parametrize("c", [2, 8, 16])
@pytest.mark.parametrize("lens,H,W", PRICED_PLAN_CASES)
def test_device_priced_plan_equals_oracle(lens, H, W, c):
    announce(f"device priced plan lens[:4]={lens[:4]} B={len(lens)} H={H} W={W} c={c}")
    assert np.array_equal(_device_plan(lens, H, W, entry_price=c), build_plan(lens, H, W, c))


def test_device_priced_plan_random_batches():
    rng = np.random.default_rng(321)
    for i in range(40):
        B = int(rng.integers(1, 70))
        H = int(rng.integers(1, 9))
        W = int(rng.integers(1, 1200))
        c = int(rng.choice([1, 2, 4, 8, 16, 64]))
        lens = rng.integers(0, 20000, size=B)
        lens[rng.random(B) < 0.2] = 0
        announce(f"device priced plan random #{i} B={B} H={H} W={W} c={c}")
        assert np.array_equal(_device_plan(lens, H, W, entry_price=c), build_plan(lens, H, W, c)), \
            (lens.tolist(), H, W, c)


@pytest.mark.parametrize("lens,H,W,c", [
    ([64 * (2 ** 25 - 1)], 16, 64, 3),                      # C = 2^31 - 16: the largest priced cost
    ([64 * (2 ** 25 - 1)], 16, 64, 4),                      # C = 2^31: declined
    ([2 ** 28 - 1, 5, 2 ** 27 + 13, 0] * 4, 8, 2047, 16),   # C near 2^29.6, large quotients
    ([64 * 2047 - 1, 1, 1, 1], 1, 2048, 8),                 # W just above T: declined
])
def test_device_priced_plan_extremes(lens, H, W, c):
    """Too many tiles for the float64 oracle's walk: the device plan against the
    host planner, which equals the oracle on every smaller case."""
    announce(f"device priced plan extreme B={len(lens)} H={H} W={W} c={c}")
    host = hd.hpc_decode_plan(np.asarray(lens, dtype=np.int32), H, W, entry_price=c)
    assert np.array_equal(_device_plan(lens, H, W, entry_price=c), host)


@pytest.mark.parametrize("cfg,W,c", [(5, 512, 8), (5, 256, 8), (4, 256, 4), (4, 252, 8), (2, 256, 16),
                                     (3, 256, 8), (1, 3, 4)])
def test_priced_step_equals_host_planned(cfg, W, c):
    """The device-scheduled step with an entry price against the host-planned
    step of the oracle's priced plan (bitwise on unsplit units) and against
    the float64 oracle."""
    inp = workload_inputs(cfg, poison=True)
    dev = to_device(inp)
    announce(f"priced device step vs host plan, workload {cfg}, W={W}, c={c}")
    plan = build_plan(inp.seq_lens.numpy(), inp.num_kv_heads, W, c)
    a = run_step(inp, W, dev, entry_price=c)
    b = run_hip_plan(inp, plan, dev)
    assert_same_as_host_planned(inp, W, a, b, plan=plan)
    compare(inp, a, run_oracle(inp), f"priced device step workload {cfg} W={W} c={c}")


@pytest.mark.parametrize("lens,hq,hkv,W", [
    ([0, 37, 0, 1], 8, 1, 3), ([63, 64, 65, 127, 128, 129], 8, 1, 5), ([300, 1000, 7], 12, 3, 11),
    ([4000, 17], 64, 8, 64), ([0, 5, 0, 130] * 16 + [64], 8, 1, 40), ([64] * 64, 16, 2, 300),
])
@pytest.mark.parametrize("fused", [False, True])
def test_priced_step_edge_shapes(lens, hq, hkv, W, fused):
    inp = make_inputs(lens, hq, hkv, "bf16", seed=len(lens) + hq + 1, poison=True)
    announce(f"priced device step edge lens[:4]={lens[:4]} B={len(lens)} hq={hq} hkv={hkv} W={W} fused={fused}")
    dev = to_device(inp)
    a = run_hip_step(inp, W, dev, fused_merge=fused, entry_price=16)
    plan = build_plan(inp.seq_lens.numpy(), hkv, W, 16)
    b = run_hip_plan(inp, plan, dev)
    if not fused:
        assert_same_as_host_planned(inp, W, a, b, plan=plan)
    compare(inp, a, run_oracle(inp), "priced device step edge")


def test_priced_repeated_steps_with_changing_splits():
    """One workspace reused across priced steps whose lengths change which
    units are split, with the in-kernel merge (its counters must return to
    zero every step)."""
    base = make_inputs([7000, 300, 65, 4000], 16, 2, "fp8_e4m3", seed=19, max_pages_per_seq=130)
    dev = to_device(base)
    ws = torch.zeros(hd.hpc_decode_step_workspace_size(4, 16, 2, 64), dtype=torch.uint8, device="cuda")
    for i, lens in enumerate(([7000, 300, 65, 4000], [7001, 0, 66, 4100], [8000, 1, 64, 8300],
                              [100, 200, 300, 400], [0, 0, 0, 0], [7000, 300, 65, 4000])):
        for fused in (True, False):
            announce(f"priced repeated step {i} fused={fused} lens={lens}")
            dev["sl"].copy_(torch.tensor(lens, dtype=torch.int32))
            base.seq_lens = torch.tensor(lens, dtype=torch.int32)
            got = run_hip_step(base, 64, dev, fused_merge=fused, workspace=ws, entry_price=8)
            compare(base, got, run_oracle(base), f"priced step {i} fused={fused}")
