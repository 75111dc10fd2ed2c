"""The tracing window (hpc_decode_trace_start / stop) on the GPU: a traced
step still matches the oracle; every worker's stamps are in order; the
recorded tile and entry counts agree with the schedule (the host planner's
words for the same lengths and W); nothing is recorded outside the window."""
import numpy as np
import pytest
import torch

import load_balanced_paged_step_amd as hd
from workloads import workload_inputs

from decode_harness import announce, compare, run_hip_plan, run_hip_step, run_oracle, to_device

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A5A5A5A5A5A5A


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hd.lib()


def _buffer(W):
    return torch.full((8 * W,), SENTINEL - (1 << 64) if SENTINEL >= 1 << 63 else SENTINEL, dtype=torch.int64,
                      device="cuda")


@pytest.mark.parametrize("cfg,W", [(4, 252), (1, 7), (5, 512)])
def test_traced_device_step(cfg, W):
    announce(f"traced device step, workload {cfg}, W={W}")
    inp = workload_inputs(cfg, poison=True)
    dev = to_device(inp)
    buf = _buffer(W)
    hd.hpc_decode_trace_start(buf)
    try:
        got = run_hip_step(inp, W, dev)
    finally:
        hd.hpc_decode_trace_stop()
    compare(inp, got, run_oracle(inp), f"traced workload {cfg} W={W}")
    st = buf.cpu().numpy().view(np.uint64).reshape(W, 8)
    words = hd.hpc_decode_plan(inp.seq_lens.numpy(), inp.num_kv_heads, W)
    wp = words[16:16 + W + 1]
    entries = np.diff(wp)
    T = int(words[4])
    tiles = np.array([(w + 1) * T // W - w * T // W for w in range(W)])
    busy = tiles > 0
    assert np.array_equal(st[busy, 5], tiles[busy])
    assert np.array_equal(st[busy, 6], entries[busy])
    # placement word: the XCC id is below 8 on MI355X
    xcc = st[busy, 7] >> np.uint64(32)
    assert np.all(xcc < 8)
    t = st[busy, :5].astype(np.int64)
    assert np.all(t > 0) and np.all(np.diff(t, axis=1) >= 0), "stamps out of order"
    # a step takes microseconds: at 100 MHz, under 1 ms between entry and end
    assert np.all(t[:, 4] - t[:, 0] < 100_000)
    assert np.all(st[~busy] == SENTINEL), "workers without tiles write nothing"


def test_traced_host_plan_and_window_off():
    inp = workload_inputs(4, poison=True)
    dev = to_device(inp)
    W = 256
    announce("traced host-planned step, then a step outside the window")
    buf = _buffer(W)
    hd.hpc_decode_trace_start(buf)
    try:
        got = run_hip_plan(inp, hd.hpc_decode_plan(inp.seq_lens.numpy(), 1, W), dev)
    finally:
        hd.hpc_decode_trace_stop()
    compare(inp, got, run_oracle(inp), "traced host plan W=256")
    st = buf.cpu().numpy().view(np.uint64).reshape(W, 8)
    assert np.all(st[:, 5] == 0)                        # no tile count with a host plan
    assert np.all(np.diff(st[:, :5].astype(np.int64), axis=1) >= 0)
    before = buf.clone()
    run_hip_step(inp, W, dev)                           # window off: the buffer is left alone
    assert torch.equal(buf, before)


def test_a_small_buffer_records_nothing():
    inp = workload_inputs(1)
    buf = _buffer(4)                                    # room for 4 workers, the step has 7
    hd.hpc_decode_trace_start(buf)
    try:
        run_hip_step(inp, 7)
    finally:
        hd.hpc_decode_trace_stop()
    assert np.all(buf.cpu().numpy().view(np.uint64) == SENTINEL)
