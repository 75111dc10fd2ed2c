"""The seeded input generator: determinism, shapes, block-table structure, poison placement."""
import numpy as np
import torch

from workloads import make_inputs, workload_inputs, draw_loguniform_lengths, WORKLOADS, PAGE


def test_deterministic_and_seed_sensitive():
    a = make_inputs([37, 200], 8, 1, "bf16", seed=1)
    b = make_inputs([37, 200], 8, 1, "bf16", seed=1)
    c = make_inputs([37, 200], 8, 1, "bf16", seed=2)
    assert torch.equal(a.k_cache.view(torch.int16), b.k_cache.view(torch.int16))
    assert not torch.equal(a.k_cache.view(torch.int16), c.k_cache.view(torch.int16))


def test_block_table_is_a_permutation_of_pages():
    inp = make_inputs([37, 64, 130, 200], 8, 1, "bf16", seed=1)
    n = [(L + PAGE - 1) // PAGE for L in (37, 64, 130, 200)]
    used = np.concatenate([inp.block_table[b, :n[b]].numpy() for b in range(4)])
    assert sorted(used.tolist()) == list(range(sum(n))) == list(range(inp.num_pages))


def test_poison_layout():
    inp = make_inputs([37, 64], 8, 1, "bf16", seed=1, poison=True, max_pages_per_seq=3)
    bt = inp.block_table.numpy()
    poison_page = inp.num_pages - 1
    assert bt[0, 1] == poison_page and bt[0, 2] == poison_page and bt[1, 1] == poison_page
    k = inp.k_cache.to(torch.float32)
    assert torch.isnan(k[poison_page]).all()
    assert torch.isnan(k[bt[0, 0], :, 37:]).all() and not torch.isnan(k[bt[0, 0], :, :37]).any()
    assert not torch.isnan(k[bt[1, 0]]).any()


def test_fp8_scales_and_range():
    inp = make_inputs([300], 16, 2, "fp8_e4m3", seed=3)
    assert inp.k_cache.dtype == torch.float8_e4m3fn
    deq = inp.k_cache.to(torch.float32)
    assert deq.abs().max().item() <= 448.0 and deq.abs().max().item() >= 400.0
    assert 0.005 < inp.k_scale < 0.02 and 0.005 < inp.v_scale < 0.02


def test_loguniform_lengths_in_range():
    rng = np.random.default_rng(5)
    lens = draw_loguniform_lengths(rng, 10000, 128, 65536)
    assert lens.min() >= 128 and lens.max() <= 65536
    assert abs(np.median(np.log(lens)) - 0.5 * (np.log(128) + np.log(65536))) < 0.1


def test_named_workloads_shapes():
    inp = workload_inputs(1)
    assert inp.q.shape == (4, 8, 128) and inp.k_cache.shape == (9, 1, 64, 128)
    assert inp.algorithmic_bytes() == 237056
    assert WORKLOADS[4].seq_lens[0] == 131072 and len(WORKLOADS[4].seq_lens) == 32


def test_all_empty_batch_has_a_page():
    inp = make_inputs([0, 0], 8, 1, "bf16", seed=1)
    assert inp.num_pages == 1 and inp.block_table.shape == (2, 1)
