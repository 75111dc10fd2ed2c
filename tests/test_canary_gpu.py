"""Stray-write guard: every buffer the step writes (out, lse and the
workspace) sits between two 4 KiB canary bands, and after the step the
bands must hold their fill byte unchanged.  A write past either end of any
of them (an off-by-one slot, a padded head, a record of a unit that does not
exist) would change a band.  The results inside are checked against the
float64 oracle as usual.

Paths: the device-scheduled step with both tile maths and with the merge in
the decode kernel, and the host-planned step (balanced and static plans),
on the skewed batch, the fp8 64q/8kv batch and a batch with empty and
one-token sequences.
"""
import numpy as np
import pytest
import torch

import load_balanced_paged_step_amd as hd
from workloads import make_inputs, workload_inputs

from decode_harness import announce, compare, run_oracle, to_device

pytestmark = pytest.mark.gpu

BAND = 4096
FILL = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hd.lib()


class Banded:
    """A device buffer of `nbytes` between two canary bands."""

    def __init__(self, nbytes, dtype, shape, zero=False):
        self.nbytes = int(nbytes)
        self.raw = torch.full((BAND + self.nbytes + BAND,), FILL, dtype=torch.uint8, device="cuda")
        inner = self.raw[BAND:BAND + self.nbytes]
        if zero:
            inner.zero_()
        self.t = inner.view(dtype).view(shape) if shape is not None else inner

    def check(self, what):
        torch.cuda.synchronize()
        lo = self.raw[:BAND].cpu().numpy()
        hi = self.raw[BAND + self.nbytes:].cpu().numpy()
        for name, band in (("before", lo), ("after", hi)):
            bad = np.nonzero(band != FILL)[0]
            assert bad.size == 0, (f"{what}: {bad.size} bytes of the band {name} the buffer were written "
                                   f"(first at band offset {int(bad[0])})")


def _outputs(inp):
    B, Hq = inp.batch, inp.num_q_heads
    out = Banded(B * Hq * 128 * 2, torch.bfloat16, (B, Hq, 128))
    lse = Banded(B * Hq * 4, torch.float32, (B, Hq))
    return out, lse


def _np(out, lse):
    return out.t.float().cpu().numpy().astype(np.float64), lse.t.cpu().numpy().astype(np.float64)


def _device_step(inp, dev, W, tile_math="mfma", fused=False):
    nb = hd.hpc_decode_step_workspace_size(inp.batch, inp.num_q_heads, inp.num_kv_heads, W)
    ws = Banded(nb, torch.uint8, None, zero=True)
    out, lse = _outputs(inp)
    hd.hpc_decode_step(dev["q"], dev["k"], dev["v"], dev["bt"], dev["sl"], ws.t, out.t, lse.t,
                       num_kv_heads=inp.num_kv_heads, n_workers=W, sm_scale=inp.sm_scale, k_scale=inp.k_scale,
                       v_scale=inp.v_scale, tile_math=tile_math, fused_merge=fused)
    return ws, out, lse


def _host_plan(inp, dev, plan):
    plan_host = np.ascontiguousarray(plan, dtype=np.int32)
    plan_dev = torch.from_numpy(plan_host).cuda()
    nb = hd.hpc_decode_workspace_size(plan_host, inp.num_q_heads, inp.num_kv_heads)
    ws = Banded(max(nb, 1), torch.uint8, None)
    out, lse = _outputs(inp)
    hd.hpc_decode_attn(dev["q"], dev["k"], dev["v"], dev["bt"], dev["sl"], plan_host, plan_dev,
                       ws.t if nb > 0 else None, out.t, lse.t, num_kv_heads=inp.num_kv_heads,
                       sm_scale=inp.sm_scale, k_scale=inp.k_scale, v_scale=inp.v_scale)
    return ws, out, lse


CASES = {
    "skewed": lambda: workload_inputs(4, poison=True),
    "fp8": lambda: workload_inputs(5, poison=True),
    "edge": lambda: make_inputs([0, 1, 65, 3000, 0, 64, 129], 16, 2, "bf16", seed=33, poison=True),
}


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("W", [7, 256])
def test_bands_intact(case, W):
    inp = CASES[case]()
    dev = to_device(inp)
    ref = run_oracle(inp)
    G = inp.num_q_heads // inp.num_kv_heads
    runs = [("device mfma", lambda: _device_step(inp, dev, W)),
            ("device fused merge", lambda: _device_step(inp, dev, W, fused=True)),
            ("host plan", lambda: _host_plan(inp, dev, hd.hpc_decode_plan(inp.seq_lens.numpy(),
                                                                          inp.num_kv_heads, W))),
            ("static plan S=4", lambda: _host_plan(inp, dev, hd.hpc_decode_plan_static(
                inp.seq_lens.numpy(), inp.num_kv_heads, 4)))]
    if G <= hd.VALU_MAX_GROUP:
        runs.append(("device valu", lambda: _device_step(inp, dev, W, tile_math="valu")))
    for name, run in runs:
        what = f"{case} W={W} {name}"
        announce(f"canary bands, {what}")
        ws, out, lse = run()
        for buf, part in ((ws, "workspace"), (out, "out"), (lse, "lse")):
            buf.check(f"{what} {part}")
        compare(inp, _np(out, lse), ref, what)
