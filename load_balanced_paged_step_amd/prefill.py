"""Python binding of causal prefill / extend attention over the paged cache
(``include/hpc_prefill.h``).

Argument marshalling only: the work-list planner runs in the library's C++
code and the attention and the merge of cut units in its HIP kernels.
Method context: "vLLM x HPC-Ops ...", §Attention Across Prefill, Extend and
Decode Shapes (the shapes), §Attention Backend: Dynamic Load-Balanced
Scheduling (the balancing the planner can apply).
"""

from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _lib
from ._lib import lib

__all__ = ["hpc_prefill_units", "hpc_prefill_plan_size", "hpc_prefill_plan", "hpc_prefill_workspace_size",
           "hpc_prefill_attn", "hpc_prefill_check", "PrefillStep", "ENTRY_WORDS", "MERGE_WORDS"]

_I32P = ctypes.POINTER(ctypes.c_int32)
ENTRY_WORDS = 8
MERGE_WORDS = 8


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


def hpc_prefill_plan_size(q_start, num_kv_heads: int, n_workers: int = 0) -> int:
    qs = _host_i32(q_start)
    return _lib.check(lib().hpc_prefill_plan_size(qs.ctypes.data_as(_I32P), qs.shape[0] - 1, num_kv_heads,
                                                  n_workers), "hpc_prefill_plan_size")


def hpc_prefill_plan(q_start, seq_lens, num_kv_heads: int, max_pages_per_seq: int, n_workers: int = 0,
                     min_share_tiles: int = 1):
    """(words, (n_entries, n_merge, n_partials)): entries [n_entries][8] =
    (b, j, h, tiles, t0, t1, slot, 0) longest first, then merge records
    [n_merge][8] = (b, j, h, S, base, 0, 0, 0)."""
    qs, sl = _host_i32(q_start), _host_i32(seq_lens)
    cap = hpc_prefill_plan_size(qs, num_kv_heads, n_workers)
    words = np.zeros(max(cap, 1), dtype=np.int32)
    counts = np.zeros(3, dtype=np.int32)
    _lib.check(lib().hpc_prefill_plan(qs.ctypes.data_as(_I32P), sl.ctypes.data_as(_I32P), sl.shape[0], num_kv_heads,
                                      max_pages_per_seq, n_workers, min_share_tiles, words.ctypes.data_as(_I32P), cap,
                                      counts.ctypes.data_as(_I32P)), "hpc_prefill_plan")
    n_e, n_m, n_p = (int(x) for x in counts)
    return words[:ENTRY_WORDS * n_e + MERGE_WORDS * n_m].copy(), (n_e, n_m, n_p)


def hpc_prefill_workspace_size(n_partials: int, num_q_heads: int, num_kv_heads: int) -> int:
    return _lib.check(lib().hpc_prefill_workspace_size(n_partials, num_q_heads, num_kv_heads),
                      "hpc_prefill_workspace_size")


def _dev(t, name, dtype=None, allow_none=False):
    from . import _dev_ptr
    return _dev_ptr(t, name, dtype, allow_none=allow_none)


def _attn_args(q, q_start, k_cache, v_cache, block_table, seq_lens, work_dev, counts, workspace, out, lse,
               num_kv_heads, sm_scale, k_scale, v_scale):
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
    n_e, n_m, n_p = counts
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return params, [ctypes.c_int32(B), ctypes.c_int32(q.shape[0]), _dev(q, "q", bf),
                    _dev(q_start, "q_start", torch.int32), _dev(k_cache, "k_cache", (bf, f8)),
                    _dev(v_cache, "v_cache", (bf, f8)), _dev(block_table, "block_table", torch.int32),
                    _dev(seq_lens, "seq_lens", torch.int32), _dev(work_dev, "work", torch.int32, allow_none=True),
                    ctypes.c_int32(n_e), ctypes.c_int32(n_m), ctypes.c_int32(n_p),
                    _dev(workspace, "workspace", allow_none=True), ctypes.c_int64(ws_bytes),
                    _dev(out, "out", bf), _dev(lse, "lse", torch.float32)]


def hpc_prefill_check(q, q_start, k_cache, v_cache, block_table, seq_lens, work_dev, counts, workspace, out, lse, *,
                      num_kv_heads, sm_scale, k_scale=1.0, v_scale=1.0) -> int:
    params, args = _attn_args(q, q_start, k_cache, v_cache, block_table, seq_lens, work_dev, counts, workspace, out,
                              lse, num_kv_heads, sm_scale, k_scale, v_scale)
    return lib().hpc_prefill_check(ctypes.byref(params), *args)


def hpc_prefill_attn(q, q_start, k_cache, v_cache, block_table, seq_lens, work_dev, counts, workspace, out, lse, *,
                     num_kv_heads, sm_scale, k_scale=1.0, v_scale=1.0, stream=None) -> None:
    from . import _stream_handle
    params, args = _attn_args(q, q_start, k_cache, v_cache, block_table, seq_lens, work_dev, counts, workspace, out,
                              lse, num_kv_heads, sm_scale, k_scale, v_scale)
    _lib.check(lib().hpc_prefill_attn(ctypes.byref(params), *args, _stream_handle(stream)), "hpc_prefill_attn")


class PrefillStep:
    """Plans a prefill / extend step on the host (lengths known there), keeps
    the work list and the partials' workspace on the device, and launches
    the attention (and the merge of cut units).  n_workers = 0 cuts nothing;
    n_workers > 0 cuts every unit longer than 2 q, q = max(ceil(T /
    n_workers), min_share_tiles), into shares of q tiles; None (the default)
    takes two workers per compute unit of the device, the count measured
    best on MI355X (two workgroups of one group fit a CU)."""

    #: shares shorter than this many tiles cost more in partial writes and the
    #: merge than they save (measured on the q512 prompts, whose units are
    #: at most 8 tiles)
    MIN_SHARE_TILES = 16

    def __init__(self, q_start_host, seq_lens_host, num_q_heads: int, num_kv_heads: int, max_pages_per_seq: int,
                 n_workers: int | None = None, min_share_tiles: int | None = None, device="cuda"):
        if min_share_tiles is None:
            min_share_tiles = self.MIN_SHARE_TILES
        if n_workers is None:
            n_workers = 2 * torch.cuda.get_device_properties(torch.device(device)).multi_processor_count
        self.words, self.counts = hpc_prefill_plan(q_start_host, seq_lens_host, num_kv_heads, max_pages_per_seq,
                                                   n_workers, min_share_tiles)
        self.n_entries, self.n_merge, self.n_partials = self.counts
        self.work_dev = torch.from_numpy(self.words).to(device) if self.words.size else None
        nb = hpc_prefill_workspace_size(self.n_partials, num_q_heads, num_kv_heads)
        self.workspace = torch.empty(nb, dtype=torch.uint8, device=device) if nb > 0 else None
        self.num_kv_heads = num_kv_heads

    @property
    def entries(self) -> np.ndarray:
        return self.words[:ENTRY_WORDS * self.n_entries].reshape(-1, ENTRY_WORDS)

    @property
    def merge(self) -> np.ndarray:
        return self.words[ENTRY_WORDS * self.n_entries:].reshape(-1, MERGE_WORDS)

    def bind(self, q, q_start, k_cache, v_cache, block_table, seq_lens, out, lse, *, sm_scale, k_scale=1.0,
             v_scale=1.0, stream=None):
        """A callable that issues this step's launches with their arguments
        marshalled once (the tensors must stay alive and unchanged in shape)."""
        from . import _stream_handle
        params, args = _attn_args(q, q_start, k_cache, v_cache, block_table, seq_lens, self.work_dev, self.counts,
                                  self.workspace, out, lse, self.num_kv_heads, sm_scale, k_scale, v_scale)
        full = (ctypes.byref(params), *args, _stream_handle(stream))
        _lib.check(lib().hpc_prefill_check(*full[:-1]), "PrefillStep.bind")
        fn = lib().hpc_prefill_attn
        keep = (params, q, q_start, k_cache, v_cache, block_table, seq_lens, out, lse, self.work_dev, self.workspace)

        def launch() -> None:
            status = fn(*full)
            if status:
                _lib.check(status, "hpc_prefill_attn")
        launch.keep = keep
        return launch

    def __call__(self, q, q_start, k_cache, v_cache, block_table, seq_lens, out, lse, *, sm_scale, k_scale=1.0,
                 v_scale=1.0, stream=None) -> None:
        hpc_prefill_attn(q, q_start, k_cache, v_cache, block_table, seq_lens, self.work_dev, self.counts,
                         self.workspace, out, lse, num_kv_heads=self.num_kv_heads, sm_scale=sm_scale,
                         k_scale=k_scale, v_scale=v_scale, stream=stream)
