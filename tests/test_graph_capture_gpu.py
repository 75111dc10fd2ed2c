"""The device-scheduled step captured in a HIP graph: the schedule is read
from the lengths on the device at every replay, so one captured step serves
every step's lengths.  Replays are interleaved with eager work and host
synchronisation, and every replay is checked against the eager step (bitwise:
same kernels, same schedule) and against the float64 oracle, for each tile
math and merge mode."""
import numpy as np
import pytest
import torch

import load_balanced_paged_step_amd as hd
from workloads import make_inputs

from decode_harness import announce, compare, run_oracle, to_device

pytestmark = pytest.mark.gpu


def _np(out, lse):
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("mode", ["mfma", "mfma+fused_merge", "valu", "valu+fused_merge", "mfma+price"])
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_graph_replays_match_eager_over_changing_lengths(kv, mode):
    """Also with the VALU tile math and with the in-kernel merge, whose
    per-unit arrival counts live in the workspace across replays (each step
    leaves them at zero; its last arriver always folds the partials in the
    same order, so replays stay bitwise equal to eager steps)."""
    tile_math = "valu" if mode.startswith("valu") else "mfma"
    fused = mode.endswith("fused_merge")
    price = 8 if mode.endswith("price") else 0
    hq, hkv, W = (16, 2, 64) if kv == "bf16" else (64, 8, 48)
    base = make_inputs([7000, 300, 65, 4000], hq, hkv, kv, seed=29, max_pages_per_seq=130)
    dev = to_device(base)
    sl = dev["sl"]
    out = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    launch = hd.StepLauncher(dev["q"], dev["k"], dev["v"], dev["bt"], sl, out, lse, num_kv_heads=hkv, n_workers=W,
                             sm_scale=base.sm_scale, k_scale=base.k_scale, v_scale=base.v_scale, stream=s,
                             tile_math=tile_math, fused_merge=fused, entry_price=price)
    with torch.cuda.stream(s):
        launch()                                  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    announce(f"graph capture of the device step ({kv}, {mode})")
    with torch.cuda.graph(g, stream=s):
        launch()
    torch.cuda.synchronize()
    steps = ([7000, 300, 65, 4000], [7001, 0, 66, 4100], [8000, 1, 64, 8300], [100, 200, 300, 400],
             [0, 0, 0, 0], [7000, 300, 65, 4000])
    for i, lens in enumerate(steps):
        announce(f"graph replay {i} lens={lens} ({kv}, {mode})")
        sl.copy_(torch.tensor(lens, dtype=torch.int32))
        torch.cuda.synchronize()
        # eager reference on the same buffers
        with torch.cuda.stream(s):
            launch()
        torch.cuda.synchronize()
        ref = _np(out, lse)
        out.fill_(float("nan"))                   # eager work between the eager step and the replay
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _np(out, lse)
        assert np.array_equal(got[0], ref[0], equal_nan=False) and np.array_equal(got[1], ref[1]), \
            f"replay {i} differs from the eager step ({mode})"
        base.seq_lens = torch.tensor(lens, dtype=torch.int32)
        compare(base, got, run_oracle(base), f"graph replay {i} ({kv}, {mode})")
