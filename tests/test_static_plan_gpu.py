"""The static split-KV schedule (C++ planner) run through hpc_decode_attn,
against the float64 oracle; same tolerances as the balanced schedule
(max|out - oracle| <= 1e-2 max|V| bf16, 3e-2 max|V| fp8; per unit
max|out_u - oracle_u| <= 1e-2 max|oracle_u| + 1e-6; lse 1e-3 / 1e-2)."""
import numpy as np
import pytest
import torch

import load_balanced_paged_step_amd as hd
from oracle.plan import build_static_plan, static_split_count
from workloads import make_inputs, workload_inputs

from decode_harness import announce, compare, run_hip_plan, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hd.lib()


def _static(inp, S):
    plan = hd.hpc_decode_plan_static(inp.seq_lens.numpy(), inp.num_kv_heads, S)
    assert np.array_equal(plan, build_static_plan(inp.seq_lens.numpy(), inp.num_kv_heads, S))
    return plan


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
@pytest.mark.parametrize("S", [1, 3, 8, 128, "rule"])
def test_static_plans_bf16(cfg, S):
    inp = workload_inputs(cfg, poison=True)
    if S == "rule":
        S = static_split_count(inp.seq_lens.numpy(), inp.num_kv_heads, 256)
    announce(f"static split-KV, workload {cfg}, poisoned, S={S}")
    compare(inp, run_hip_plan(inp, _static(inp, S)), run_oracle(inp), f"static S={S} workload {cfg}")


def test_static_plan_fp8_full_heads():
    inp = workload_inputs(5, poison=True)
    S = static_split_count(inp.seq_lens.numpy(), inp.num_kv_heads, 256)
    announce(f"static split-KV, workload 5, poisoned, S={S}")
    compare(inp, run_hip_plan(inp, _static(inp, S)), run_oracle(inp), f"static S={S} workload 5")


def test_static_plan_with_empty_sequences():
    inp = make_inputs([0, 700, 0, 65, 1], 16, 2, "bf16", seed=21, poison=True)
    announce("static split-KV, empty sequences, S=4")
    compare(inp, run_hip_plan(inp, _static(inp, 4)), run_oracle(inp), "static with empties")
