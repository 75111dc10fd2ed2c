"""GPU tests of the one-call host-planned step (hpc_decode_plan_attn): the
native planner, the queued plan upload and the kernels in one C call."""
import ctypes

import numpy as np
import pytest
import torch

import load_balanced_paged_step_amd as hd
from workloads import make_inputs

from decode_harness import announce, compare, run_hip, run_oracle, to_device

pytestmark = pytest.mark.gpu


def _np(out, lse):
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("lens,hq,hkv,W,kv", [
    ([37, 64, 130, 200], 8, 1, 4, "bf16"), ([7000, 300, 0, 4000], 16, 2, 64, "bf16"),
    ([3000, 65, 129], 64, 8, 40, "fp8_e4m3"),
])
def test_plan_attn_equals_attn(lens, hq, hkv, W, kv):
    """Same plan, same kernels: bitwise the result of hpc_decode_plan + hpc_decode_attn."""
    inp = make_inputs(lens, hq, hkv, kv, seed=len(lens) + W, poison=True)
    announce(f"plan_attn lens={lens} hq={hq} hkv={hkv} W={W} {kv}")
    dev = to_device(inp)
    out = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    cap = hd.hpc_decode_plan_size(len(lens), hkv, W)
    host = torch.empty(cap, dtype=torch.int32, pin_memory=True)
    plan_dev = torch.empty(cap, dtype=torch.int32, device="cuda")
    ws = torch.empty(hd.hpc_decode_plan_workspace_bound(len(lens), hq, hkv, W), dtype=torch.uint8, device="cuda")
    words = hd.hpc_decode_plan_attn(inp.seq_lens, host, plan_dev, dev["q"], dev["k"], dev["v"], dev["bt"],
                                    dev["sl"], ws, out, lse, num_kv_heads=hkv, n_workers=W,
                                    sm_scale=inp.sm_scale, k_scale=inp.k_scale, v_scale=inp.v_scale)
    torch.cuda.synchronize()
    got = _np(out, lse)
    assert np.array_equal(words, hd.hpc_decode_plan(inp.seq_lens, hkv, W))
    assert np.array_equal(plan_dev[:words.shape[0]].cpu().numpy(), words)
    ref = run_hip(inp, W, dev)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
    compare(inp, got, run_oracle(inp), "plan_attn")


@pytest.mark.parametrize("lens,hq,hkv,W,kv,c", [
    ([7000, 300, 0, 4000], 16, 2, 64, "bf16", 8), ([3000, 65, 129, 5000], 64, 8, 40, "fp8_e4m3", 16),
])
def test_plan_attn_with_entry_price(lens, hq, hkv, W, kv, c):
    """The one-call step plans with params.entry_price: its plan words are
    the priced planner's (the price applied, header word 9), and the result
    is bitwise that of hpc_decode_attn with the oracle's priced plan."""
    from oracle import build_plan
    from decode_harness import run_hip_plan
    inp = make_inputs(lens, hq, hkv, kv, seed=len(lens) + W + c, poison=True)
    announce(f"plan_attn priced lens={lens} hq={hq} hkv={hkv} W={W} {kv} c={c}")
    dev = to_device(inp)
    out = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    cap = hd.hpc_decode_plan_size(len(lens), hkv, W)
    host = torch.empty(cap, dtype=torch.int32, pin_memory=True)
    plan_dev = torch.empty(cap, dtype=torch.int32, device="cuda")
    ws = torch.empty(hd.hpc_decode_plan_workspace_bound(len(lens), hq, hkv, W), dtype=torch.uint8, device="cuda")
    words = hd.hpc_decode_plan_attn(inp.seq_lens, host, plan_dev, dev["q"], dev["k"], dev["v"], dev["bt"],
                                    dev["sl"], ws, out, lse, num_kv_heads=hkv, n_workers=W,
                                    sm_scale=inp.sm_scale, k_scale=inp.k_scale, v_scale=inp.v_scale, entry_price=c)
    torch.cuda.synchronize()
    got = _np(out, lse)
    plan = build_plan(inp.seq_lens.numpy(), hkv, W, c)
    assert int(plan[9]) == c and np.array_equal(words, plan)
    ref = run_hip_plan(inp, plan, dev)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
    compare(inp, got, run_oracle(inp), "plan_attn priced")


@pytest.mark.parametrize("in_place", [False, True])
def test_launcher_runs_ahead_over_changing_lengths(in_place):
    """Steps queued back to back with no host synchronisation, each with other
    lengths: the two pinned plan buffers are reused in turn while earlier
    uploads (or, in place, earlier kernels reading them) may still be queued,
    and every step still matches the oracle."""
    base = make_inputs([7000, 300, 65, 4000], 16, 2, "bf16", seed=23, max_pages_per_seq=130)
    dev = to_device(base)
    out = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    sl = dev["sl"]
    launch = hd.PlannedStepLauncher(dev["q"], dev["k"], dev["v"], dev["bt"], sl, out, lse, num_kv_heads=2,
                                    n_workers=64, sm_scale=base.sm_scale, in_place=in_place)
    steps = ([7000, 300, 65, 4000], [7001, 0, 66, 4100], [8000, 1, 64, 8300], [100, 200, 300, 400],
             [0, 0, 0, 0], [64, 8320, 1, 5], [7000, 300, 65, 4000])
    lens_dev = [torch.tensor(x, dtype=torch.int32).pin_memory() for x in steps]
    results = []
    announce(f"planned launcher (in place: {in_place}), {len(steps)} steps queued")
    for x, xd in zip(steps, lens_dev):
        sl.copy_(xd, non_blocking=True)
        launch(np.asarray(x, dtype=np.int32))
        results.append((out.clone(), lse.clone()))
    torch.cuda.synchronize()
    assert np.array_equal(launch.plan_host, hd.hpc_decode_plan(steps[-1], 2, 64))
    for i, (x, (o, l)) in enumerate(zip(steps, results)):
        base.seq_lens = torch.tensor(x, dtype=torch.int32)
        compare(base, _np(o, l), run_oracle(base), f"queued step {i} lens={x}")


def test_launcher_rejects_wrong_batch():
    inp = make_inputs([100, 200], 8, 1, "bf16", seed=5)
    dev = to_device(inp)
    out = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    launch = hd.PlannedStepLauncher(dev["q"], dev["k"], dev["v"], dev["bt"], dev["sl"], out, lse,
                                    num_kv_heads=1, n_workers=8, sm_scale=inp.sm_scale)
    with pytest.raises(ValueError):
        launch(np.asarray([1, 2, 3], dtype=np.int32))
    with pytest.raises(hd.HpcDecodeError):
        launch(np.asarray([100, 10_000], dtype=np.int32))      # beyond the block table: checked on the host
    launch(inp.seq_lens.numpy())
    torch.cuda.synchronize()
    compare(inp, _np(out, lse), run_oracle(inp), "after rejected calls")


def test_plan_in_place_equals_copied_plan():
    """The kernels reading the plan from pinned host memory give bitwise the
    result of the uploaded plan; a host pointer that is not pinned is refused."""
    inp = make_inputs([7000, 300, 0, 4000, 129], 16, 2, "bf16", seed=31, poison=True)
    announce("plan read in place from pinned memory")
    dev = to_device(inp)
    cap = hd.hpc_decode_plan_size(inp.batch, 2, 48)
    ws = torch.empty(hd.hpc_decode_plan_workspace_bound(inp.batch, 16, 2, 48), dtype=torch.uint8, device="cuda")
    res = []
    for in_place in (False, True):
        out = torch.empty_like(dev["q"])
        lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
        host = torch.zeros(cap, dtype=torch.int32, pin_memory=True)
        plan_dev = host if in_place else torch.empty(cap, dtype=torch.int32, device="cuda")
        params, args = hd._step_args(dev["q"], dev["k"], dev["v"], dev["bt"], dev["sl"], ws, out, lse, 2, 48,
                                     inp.sm_scale, 1.0, 1.0)
        lens = inp.seq_lens.numpy().astype(np.int32)
        st = hd.lib().hpc_decode_plan_attn(ctypes.byref(params), lens.ctypes.data, inp.batch, 48,
                                           host.data_ptr(), cap, plan_dev.data_ptr(), *args[2:],
                                           hd._stream_handle(None))
        assert st == 0, hd.hpc_status_string(st)
        torch.cuda.synchronize()
        res.append(_np(out, lse))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
    compare(inp, res[1], run_oracle(inp), "plan in place")
    pageable = np.zeros(cap, dtype=np.int32)
    st = hd.lib().hpc_decode_plan_attn(ctypes.byref(params), lens.ctypes.data, inp.batch, 48, pageable.ctypes.data,
                                       cap, pageable.ctypes.data, *args[2:], hd._stream_handle(None))
    assert st == hd.HPC_ERR_INVALID
