"""Python binding of causal prefill / extend attention over the paged cache
(``include/hpc_prefill.h``).

Argument marshalling only: the work-list planner runs in the library's C++
code and the attention in its HIP kernel.  Method context: "vLLM x HPC-Ops
...", §Attention Across Prefill, Extend and Decode Shapes.
"""

from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _lib
from ._lib import lib

__all__ = ["hpc_prefill_units", "hpc_prefill_plan", "hpc_prefill_attn", "hpc_prefill_check", "PrefillStep"]

_I32P = ctypes.POINTER(ctypes.c_int32)


def _host_i32(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        if x.device.type != "cpu":
            raise ValueError("expected a host (CPU) tensor")
        x = x.numpy()
    return np.ascontiguousarray(x, dtype=np.int32).reshape(-1)


def hpc_prefill_units(q_start, num_kv_heads: int) -> int:
    qs = _host_i32(q_start)
    return _lib.check(lib().hpc_prefill_units(qs.ctypes.data_as(_I32P), qs.shape[0] - 1, num_kv_heads),
                      "hpc_prefill_units")


def hpc_prefill_plan(q_start, seq_lens, num_kv_heads: int, max_pages_per_seq: int) -> np.ndarray:
    """The work list [n_units][4] = (sequence, query block, KV head, cost), longest first."""
    qs, sl = _host_i32(q_start), _host_i32(seq_lens)
    units = hpc_prefill_units(qs, num_kv_heads)
    work = np.zeros((max(units, 1), 4), dtype=np.int32)
    got = _lib.check(lib().hpc_prefill_plan(qs.ctypes.data_as(_I32P), sl.ctypes.data_as(_I32P), sl.shape[0],
                                            num_kv_heads, max_pages_per_seq, work.ctypes.data_as(_I32P), units),
                     "hpc_prefill_plan")
    return work[:got]


def _dev(t, name, dtype=None):
    from . import _dev_ptr
    return _dev_ptr(t, name, dtype)


def _attn_args(q, q_start, k_cache, v_cache, block_table, seq_lens, work_dev, n_units, out, lse, num_kv_heads,
               sm_scale, k_scale, v_scale):
    from . import make_params
    if q.dim() != 3 or k_cache.dim() != 4 or block_table.dim() != 2:
        raise ValueError("expected q [total,Hq,128], caches [pages,H_kv,64,128], block_table [B,max_pages]")
    B = block_table.shape[0]
    if (q_start.shape[0] != B + 1 or seq_lens.shape[0] != B or tuple(out.shape) != tuple(q.shape)
            or tuple(lse.shape) != tuple(q.shape[:2]) or tuple(k_cache.shape) != tuple(v_cache.shape)
            or k_cache.shape[1] != num_kv_heads):
        raise ValueError("prefill tensor shapes do not agree")
    params = make_params(q.shape[1], num_kv_heads, block_table.shape[1], k_cache.shape[0], k_cache.dtype, sm_scale,
                         k_scale, v_scale, head_dim=q.shape[2], page_size=k_cache.shape[2])
    bf, f8 = torch.bfloat16, torch.float8_e4m3fn
    work_ptr = _dev(work_dev, "work", torch.int32) if n_units > 0 else None
    return params, [ctypes.c_int32(B), ctypes.c_int32(q.shape[0]), _dev(q, "q", bf),
                    _dev(q_start, "q_start", torch.int32), _dev(k_cache, "k_cache", (bf, f8)),
                    _dev(v_cache, "v_cache", (bf, f8)), _dev(block_table, "block_table", torch.int32),
                    _dev(seq_lens, "seq_lens", torch.int32), work_ptr, ctypes.c_int32(n_units),
                    _dev(out, "out", bf), _dev(lse, "lse", torch.float32)]


def hpc_prefill_check(q, q_start, k_cache, v_cache, block_table, seq_lens, work_dev, n_units, out, lse, *,
                      num_kv_heads, sm_scale, k_scale=1.0, v_scale=1.0) -> int:
    params, args = _attn_args(q, q_start, k_cache, v_cache, block_table, seq_lens, work_dev, n_units, out, lse,
                              num_kv_heads, sm_scale, k_scale, v_scale)
    return lib().hpc_prefill_check(ctypes.byref(params), *args)


def hpc_prefill_attn(q, q_start, k_cache, v_cache, block_table, seq_lens, work_dev, n_units, out, lse, *,
                     num_kv_heads, sm_scale, k_scale=1.0, v_scale=1.0, stream=None) -> None:
    from . import _stream_handle
    params, args = _attn_args(q, q_start, k_cache, v_cache, block_table, seq_lens, work_dev, n_units, out, lse,
                              num_kv_heads, sm_scale, k_scale, v_scale)
    _lib.check(lib().hpc_prefill_attn(ctypes.byref(params), *args, _stream_handle(stream)), "hpc_prefill_attn")


class PrefillStep:
    """Plans a prefill / extend step on the host (lengths known there), keeps
    the work list on the device, and launches the attention."""

    def __init__(self, q_start_host, seq_lens_host, num_kv_heads: int, max_pages_per_seq: int, device="cuda"):
        self.work_host = hpc_prefill_plan(q_start_host, seq_lens_host, num_kv_heads, max_pages_per_seq)
        self.n_units = int(self.work_host.shape[0])
        self.work_dev = torch.from_numpy(self.work_host.copy()).to(device) if self.n_units else None
        self.num_kv_heads = num_kv_heads

    def bind(self, q, q_start, k_cache, v_cache, block_table, seq_lens, out, lse, *, sm_scale, k_scale=1.0,
             v_scale=1.0, stream=None):
        """A callable that issues this step's launch with its arguments
        marshalled once (the tensors must stay alive and unchanged in shape)."""
        from . import _stream_handle
        params, args = _attn_args(q, q_start, k_cache, v_cache, block_table, seq_lens, self.work_dev, self.n_units,
                                  out, lse, self.num_kv_heads, sm_scale, k_scale, v_scale)
        full = (ctypes.byref(params), *args, _stream_handle(stream))
        _lib.check(lib().hpc_prefill_check(*full[:-1]), "PrefillStep.bind")
        fn = lib().hpc_prefill_attn
        keep = (params, q, q_start, k_cache, v_cache, block_table, seq_lens, out, lse, self.work_dev)

        def launch() -> None:
            status = fn(*full)
            if status:
                _lib.check(status, "hpc_prefill_attn")
        launch.keep = keep
        return launch

    def __call__(self, q, q_start, k_cache, v_cache, block_table, seq_lens, out, lse, *, sm_scale, k_scale=1.0,
                 v_scale=1.0, stream=None) -> None:
        hpc_prefill_attn(q, q_start, k_cache, v_cache, block_table, seq_lens, self.work_dev, self.n_units, out, lse,
                         num_kv_heads=self.num_kv_heads, sm_scale=sm_scale, k_scale=k_scale, v_scale=v_scale,
                         stream=stream)
