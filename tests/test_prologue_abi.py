"""Host-side checks of hpc_decode_prologue (no GPU: every rejected call
returns before any HIP call)."""
import ctypes

import pytest

import load_balanced_paged_step_amd as hd
from load_balanced_paged_step_amd.prologue import make_prologue_params

FAKE = ctypes.c_void_p(0x1000)


def _call(params, batch=4, **null):
    names = ["q_in", "k_in", "v_in", "q_norm_w", "k_norm_w", "positions", "block_table", "k_cache", "v_cache",
             "q_out", "q_fp8"]
    ptrs = [None if null.get(n) else FAKE for n in names]
    return hd.lib().hpc_decode_prologue_check(ctypes.byref(params), batch, *ptrs)


def _params(**kw):
    base = dict(num_q_heads=8, num_kv_heads=1, max_pages_per_seq=4, num_pages=16, kv_dtype=hd.HPC_KV_BF16,
                eps=1e-6, theta=10000.0, k_scale=1.0, v_scale=1.0, q_scale=1.0)
    base.update(kw)
    return make_prologue_params(**base)


def test_accepts_a_consistent_call():
    assert _call(_params()) == hd.HPC_OK
    assert _call(_params(), q_fp8=True) == hd.HPC_OK          # q_fp8 is optional


@pytest.mark.parametrize("name", ["q_in", "k_in", "v_in", "q_norm_w", "k_norm_w", "positions", "block_table",
                                  "k_cache", "v_cache", "q_out"])
def test_null_pointers(name):
    assert _call(_params(), **{name: True}) == hd.HPC_ERR_NULL


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), hd.HPC_ERR_UNSUPPORTED),
    (dict(page_size=16), hd.HPC_ERR_UNSUPPORTED),
    (dict(kv_dtype=7), hd.HPC_ERR_UNSUPPORTED),
    (dict(num_q_heads=12, num_kv_heads=8), hd.HPC_ERR_INVALID),
    (dict(num_kv_heads=0), hd.HPC_ERR_INVALID),
    (dict(max_pages_per_seq=0), hd.HPC_ERR_INVALID),
    (dict(num_pages=0), hd.HPC_ERR_INVALID),
    (dict(eps=-1e-6), hd.HPC_ERR_INVALID),
    (dict(eps=float("nan")), hd.HPC_ERR_INVALID),
    (dict(theta=1.0), hd.HPC_ERR_INVALID),
    (dict(theta=float("inf")), hd.HPC_ERR_INVALID),
    (dict(kv_dtype=hd.HPC_KV_FP8_E4M3, k_scale=0.0), hd.HPC_ERR_INVALID),
    (dict(kv_dtype=hd.HPC_KV_FP8_E4M3, v_scale=-1.0), hd.HPC_ERR_INVALID),
    (dict(q_scale=0.0), hd.HPC_ERR_INVALID),
])
def test_bad_params(kw, code):
    assert _call(_params(**kw)) == code


def test_scales_unused_by_bf16_are_not_checked():
    assert _call(_params(k_scale=0.0, v_scale=float("nan"))) == hd.HPC_OK
    assert _call(_params(q_scale=0.0), q_fp8=True) == hd.HPC_OK    # no fp8 query: q_scale unused


def test_bad_batch():
    assert _call(_params(), batch=0) == hd.HPC_ERR_INVALID
    assert _call(_params(num_q_heads=1 << 20, num_kv_heads=1 << 10), batch=1 << 12) == hd.HPC_ERR_INVALID
