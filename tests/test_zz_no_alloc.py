"""hpc_decode_step_noalloc: the device-scheduled step with its scratch in the
library's fixed per-GPU array, called through the C ABI, against
hpc_decode_step with a freshly allocated workspace (bitwise: the two run the
same kernels on the same inputs) and against the float64 oracle.  Two calls
in a row, the second on a smaller batch, so the second finds the first's
partials and records left in the array.
"""
import ctypes

import numpy as np
import pytest
import torch

import load_balanced_paged_step_amd as hd
from workloads import make_inputs, workload_inputs

from decode_harness import announce, compare, run_oracle, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hd.lib()


def _step(inp, dev, W, noalloc, tile_math="mfma", entry_price=0):
    out = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    kw = dict(num_kv_heads=inp.num_kv_heads, n_workers=W, sm_scale=inp.sm_scale, k_scale=inp.k_scale,
              v_scale=inp.v_scale, tile_math=tile_math, entry_price=entry_price)
    if noalloc:
        hd.hpc_decode_step_noalloc(dev["q"], dev["k"], dev["v"], dev["bt"], dev["sl"], out, lse, **kw)
    else:
        nb = hd.hpc_decode_step_workspace_size(inp.batch, inp.num_q_heads, inp.num_kv_heads, W)
        ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
        hd.hpc_decode_step(dev["q"], dev["k"], dev["v"], dev["bt"], dev["sl"], ws, out, lse, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _same(a, b, what):
    assert np.array_equal(a[0], b[0]), f"{what}: outputs differ from hpc_decode_step"
    assert np.array_equal(a[1], b[1]), f"{what}: lse differ from hpc_decode_step"


@pytest.mark.parametrize("first,second,W", [
    (4, 1, 256),      # skewed 1x128K+31x4K, then the tiny batch
    (5, 3, 256),      # fp8 64q/8kv log-uniform, then 8x1024 bf16
    (4, 2, 1024),     # at 1024 workers (the largest count that fits at G = 8)
])
def test_two_calls_second_smaller(first, second, W):
    for cfg in (first, second):
        inp = workload_inputs(cfg, poison=True)
        dev = to_device(inp)
        announce(f"no-alloc step, workload {cfg}, W={W}")
        got = _step(inp, dev, W, noalloc=True)
        ref = _step(inp, dev, W, noalloc=False)
        _same(got, ref, f"workload {cfg} W={W}")
        compare(inp, got, run_oracle(inp), f"no-alloc workload {cfg} W={W}")


def test_two_priced_calls_second_smaller():
    """With the partition's entry price (the fp8 batch's rule price, 8), the
    no-allocation step equals hpc_decode_step bitwise, twice in a row."""
    for cfg in (5, 2):
        inp = workload_inputs(cfg, poison=True)
        dev = to_device(inp)
        announce(f"no-alloc priced step, workload {cfg}, W=512")
        got = _step(inp, dev, 512, noalloc=True, entry_price=8)
        _same(got, _step(inp, dev, 512, noalloc=False, entry_price=8), f"priced workload {cfg}")
        compare(inp, got, run_oracle(inp), f"no-alloc priced workload {cfg}")


def test_shrinking_edge_batches_and_valu():
    cases = [([5000, 0, 65, 1, 3000], 16, 2, "bf16", 37),
             ([129, 64], 8, 1, "fp8_e4m3", 5),
             ([1], 8, 1, "bf16", 1)]
    for i, (lens, hq, hkv, kv, W) in enumerate(cases):
        inp = make_inputs(lens, hq, hkv, kv, seed=40 + i, poison=True)
        dev = to_device(inp)
        for tm in ("mfma", "valu"):
            announce(f"no-alloc step, lens={lens} {kv} W={W} {tm}")
            got = _step(inp, dev, W, noalloc=True, tile_math=tm)
            _same(got, _step(inp, dev, W, noalloc=False, tile_math=tm), f"{lens} {tm}")
            compare(inp, got, run_oracle(inp), f"no-alloc {lens} {tm}")


def test_rejected_before_any_launch():
    inp = make_inputs([100, 200], 16, 1, "bf16", seed=2)
    dev = to_device(inp)
    out = torch.full_like(dev["q"], 7.0)
    lse = torch.full(dev["q"].shape[:2], 7.0, dtype=torch.float32, device="cuda")
    need = hd.hpc_decode_step_workspace_size(2, 16, 1, 1024)
    assert need > hd.hpc_decode_step_noalloc_max_bytes()
    with pytest.raises(hd.HpcDecodeError) as e:
        hd.hpc_decode_step_noalloc(dev["q"], dev["k"], dev["v"], dev["bt"], dev["sl"], out, lse,
                                   num_kv_heads=1, n_workers=1024, sm_scale=inp.sm_scale)
    assert e.value.status == hd.HPC_ERR_TOO_SMALL
    # the in-kernel merge keeps counts between calls: refused
    params = hd.make_params(16, 1, dev["bt"].shape[1], dev["k"].shape[0], torch.bfloat16, inp.sm_scale,
                            fused_merge=True)
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    st = hd.lib().hpc_decode_step_noalloc(ctypes.byref(params), 2, 256, vp(dev["q"]), vp(dev["k"]), vp(dev["v"]),
                                          vp(dev["bt"]), vp(dev["sl"]), vp(out), vp(lse), None)
    assert st == hd.HPC_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)
