"""Load-balanced paged GQA decode attention for AMD Instinct MI355X (gfx950).

Python binding of the C ABI in ``include/hpc_decode.h`` / ``include/hpc_probe.h``.
Each function here only checks and marshals arguments (torch tensors ->
device pointers, the current HIP stream) and calls the function of the same
name in ``libhpc_decode.so``; the schedule, the attention and the merge all
run in that library's C++ planner and HIP kernels.  PyTorch supplies device
memory and streams only.

Method: "vLLM x HPC-Ops: High-Performance Attention and MoE Backends from
Tencent Hunyuan", §Attention Backend: Dynamic Load-Balanced Scheduling.
"""

from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _lib
from ._lib import (HPC_OK, HPC_ERR_NULL, HPC_ERR_INVALID, HPC_ERR_UNSUPPORTED, HPC_ERR_PLAN_MISMATCH,
                   HPC_ERR_TOO_SMALL, HPC_ERR_HIP, HPC_KV_BF16, HPC_KV_FP8_E4M3, HEAD_DIM, PAGE,
                   MAX_GROUP, PLAN_HEADER_WORDS, HPC_TILE_MATH_MFMA, HPC_TILE_MATH_VALU, VALU_MAX_GROUP,
                   HpcDecodeError, hpc_decode_params, lib)

__all__ = [
    "hpc_decode_plan_size", "hpc_decode_plan", "hpc_decode_plan_static_size", "hpc_decode_plan_static",
    "hpc_decode_static_splits", "hpc_decode_choose_workers", "hpc_decode_pick_workers", "ENTRY_COST_TILES",
    "hpc_decode_pick_entry_price", "MAX_ENTRY_PRICE", "hpc_decode_pick_merge", "FUSED_MAX_SHARES",
    "hpc_decode_plan_words", "hpc_decode_workspace_size",
    "hpc_decode_check", "hpc_decode_attn", "hpc_status_string", "hpc_decode_profile_start",
    "hpc_decode_profile_stop", "hpc_decode_trace_start", "hpc_decode_trace_stop",
    "hpc_decode_wall_clock_hz", "hpc_probe_read", "hpc_probe_read_timed", "hpc_probe_copy", "hpc_decode_step",
    "hpc_decode_step_check", "hpc_decode_step_workspace_size", "hpc_decode_plan_device", "StepLauncher",
    "AttnLauncher",
    "hpc_decode_step_noalloc", "hpc_decode_step_noalloc_max_bytes",
    "hpc_decode_plan_workspace_bound", "hpc_decode_plan_attn", "PlannedStepLauncher",
    "DecodeStep", "HpcDecodeError",
    "kv_dtype_code", "make_params", "tile_math_code", "HPC_KV_BF16", "HPC_KV_FP8_E4M3",
    "HPC_TILE_MATH_MFMA", "HPC_TILE_MATH_VALU", "VALU_MAX_GROUP",
]

_I32P = ctypes.POINTER(ctypes.c_int32)


def _host_i32(x) -> np.ndarray:
    """A C-contiguous int32 numpy view of host data (numpy array or CPU tensor)."""
    if isinstance(x, torch.Tensor):
        if x.device.type != "cpu":
            raise ValueError("expected a host (CPU) tensor")
        x = x.numpy()
    a = np.ascontiguousarray(x, dtype=np.int32)
    return a


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(_I32P)


def _dev_ptr(t, name: str, dtype=None, allow_none: bool = False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (cuda) tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def kv_dtype_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return HPC_KV_BF16
    if dtype == torch.float8_e4m3fn:
        return HPC_KV_FP8_E4M3
    raise ValueError(f"unsupported KV-cache dtype {dtype}")


def tile_math_code(tile_math) -> int:
    """HPC_TILE_MATH_* code of ``tile_math`` ("mfma", "valu" or the code itself)."""
    if isinstance(tile_math, str):
        codes = {"mfma": HPC_TILE_MATH_MFMA, "valu": HPC_TILE_MATH_VALU}
        if tile_math not in codes:
            raise ValueError(f"tile_math must be 'mfma' or 'valu', not {tile_math!r}")
        return codes[tile_math]
    return int(tile_math)


def make_params(num_q_heads, num_kv_heads, max_pages_per_seq, num_pages, kv_dtype, sm_scale,
                k_scale=1.0, v_scale=1.0, head_dim=HEAD_DIM, page_size=PAGE,
                tile_math="mfma", fused_merge=False, entry_price=0) -> hpc_decode_params:
    code = kv_dtype if isinstance(kv_dtype, int) else kv_dtype_code(kv_dtype)
    return hpc_decode_params(int(num_q_heads), int(num_kv_heads), int(head_dim), int(page_size),
                             int(max_pages_per_seq), int(num_pages), code, float(sm_scale),
                             float(k_scale), float(v_scale), tile_math_code(tile_math), int(fused_merge),
                             int(entry_price))


# ---------------------------------------------------------------- planner ---

def hpc_decode_plan_size(batch: int, num_kv_heads: int, n_workers: int) -> int:
    return _lib.check(lib().hpc_decode_plan_size(batch, num_kv_heads, n_workers), "hpc_decode_plan_size")


def hpc_decode_plan(seq_lens, num_kv_heads: int, n_workers: int, out=None, entry_price: int = 0) -> np.ndarray:
    """Per-step schedule of host lengths ``seq_lens``; returns the used int32 words.

    ``out`` may be a preallocated host int32 buffer (numpy array or a pinned
    CPU tensor) of at least ``hpc_decode_plan_size`` words; the result is
    then a view of it.  ``entry_price`` > 0 gives the priced partition
    (``hpc_decode_plan_priced``: a unit start costs that many quarter tiles).
    """
    lens = _host_i32(seq_lens).reshape(-1)
    cap = hpc_decode_plan_size(lens.shape[0], num_kv_heads, n_workers)
    if out is None:
        buf = np.empty(cap, dtype=np.int32)
    else:
        buf = out.numpy() if isinstance(out, torch.Tensor) else out
        if buf.dtype != np.int32 or not buf.flags.c_contiguous:
            raise ValueError("plan buffer must be a contiguous int32 host buffer")
    _lib.check(lib().hpc_decode_plan_priced(_i32p(lens), lens.shape[0], num_kv_heads, n_workers, int(entry_price),
                                            _i32p(buf), buf.shape[0]), "hpc_decode_plan_priced")
    return buf[:hpc_decode_plan_words(buf)]


def hpc_decode_plan_static_size(batch: int, num_kv_heads: int, splits: int) -> int:
    return _lib.check(lib().hpc_decode_plan_static_size(batch, num_kv_heads, splits),
                      "hpc_decode_plan_static_size")


def hpc_decode_plan_static(seq_lens, num_kv_heads: int, splits: int) -> np.ndarray:
    """Static split-KV schedule (every unit cut into ``splits`` equal shares of
    its own tiles, one worker per share), in the plan word layout."""
    lens = _host_i32(seq_lens).reshape(-1)
    cap = hpc_decode_plan_static_size(lens.shape[0], num_kv_heads, splits)
    buf = np.empty(cap, dtype=np.int32)
    _lib.check(lib().hpc_decode_plan_static(_i32p(lens), lens.shape[0], num_kv_heads, splits, _i32p(buf),
                                            buf.shape[0]), "hpc_decode_plan_static")
    return buf[:hpc_decode_plan_words(buf)]


def hpc_decode_static_splits(seq_lens, num_kv_heads: int, n_cus: int, max_splits: int = 128) -> int:
    """Split count the static split-KV baseline uses for this batch."""
    lens = _host_i32(seq_lens).reshape(-1)
    return _lib.check(lib().hpc_decode_static_splits(_i32p(lens), lens.shape[0], num_kv_heads, n_cus, max_splits),
                      "hpc_decode_static_splits")


#: entry price (in tiles) of the worker-count rule (HPC_DECODE_ENTRY_COST): an
#: entry end costs about 0.6 us on MI355X against about 1.25 us per 32 KiB tile
ENTRY_COST_TILES = 0.5


def hpc_decode_choose_workers(seq_lens, num_kv_heads: int, min_workers: int, max_workers: int,
                              entry_cost: float = ENTRY_COST_TILES) -> int:
    """The worker count in [min_workers, max_workers] whose costliest worker
    (tiles + entry_cost per entry) is cheapest, ties to the larger count."""
    lens = _host_i32(seq_lens).reshape(-1)
    return _lib.check(lib().hpc_decode_choose_workers(_i32p(lens), lens.shape[0], num_kv_heads, min_workers,
                                                      max_workers, float(entry_cost)), "hpc_decode_choose_workers")


def _kv_code(kv_dtype) -> int:
    if isinstance(kv_dtype, str):
        return {"bf16": HPC_KV_BF16, "fp8_e4m3": HPC_KV_FP8_E4M3}[kv_dtype]
    if isinstance(kv_dtype, torch.dtype):
        return kv_dtype_code(kv_dtype)
    return int(kv_dtype)


def hpc_decode_pick_workers(seq_lens, num_kv_heads: int, kv_dtype, n_cus: int) -> int:
    """The worker count for a device-scheduled step on n_cus compute units:
    the worker-count rule over [n_cus / 2, n_cus], or 2 n_cus for an fp8
    cache whose partition then holds 1.5 entries per worker or more."""
    lens = _host_i32(seq_lens).reshape(-1)
    return _lib.check(lib().hpc_decode_pick_workers(_i32p(lens), lens.shape[0], num_kv_heads, _kv_code(kv_dtype),
                                                    n_cus), "hpc_decode_pick_workers")


#: largest entry price accepted (HPC_DECODE_MAX_ENTRY_PRICE), in quarter tiles
MAX_ENTRY_PRICE = 64


def hpc_decode_pick_entry_price(seq_lens, num_kv_heads: int, kv_dtype, n_workers: int) -> int:
    """The partition's entry price (quarter tiles per unit start) for a step of
    n_workers workers: among 0, 2, 4, 8 and 16, the one whose costliest
    worker prices lowest (by at least 1%), 0 when none does."""
    lens = _host_i32(seq_lens).reshape(-1)
    return _lib.check(lib().hpc_decode_pick_entry_price(_i32p(lens), lens.shape[0], num_kv_heads,
                                                        _kv_code(kv_dtype), n_workers),
                      "hpc_decode_pick_entry_price")


#: most workers per unit for which hpc_decode_pick_merge keeps the merge in the
#: decode kernel (HPC_DECODE_FUSED_MAX_SHARES)
FUSED_MAX_SHARES = 8


def hpc_decode_pick_merge(seq_lens, num_kv_heads: int, n_workers: int, entry_price: int = 0) -> bool:
    """The merge mode of a device-scheduled step (``fused_merge``): True
    (merge in the decode kernel) when no (sequence, KV head) unit of the
    step's partition is split, or when the batch has no more tiles than
    workers and no unit is shared by more than FUSED_MAX_SHARES workers;
    False (merge kernel) otherwise."""
    lens = _host_i32(seq_lens).reshape(-1)
    return bool(_lib.check(lib().hpc_decode_pick_merge(_i32p(lens), lens.shape[0], num_kv_heads, n_workers,
                                                       entry_price), "hpc_decode_pick_merge"))


def hpc_decode_plan_words(plan) -> int:
    a = _host_i32(plan) if not isinstance(plan, np.ndarray) else plan
    return _lib.check(lib().hpc_decode_plan_words(_i32p(a)), "hpc_decode_plan_words")


def hpc_decode_workspace_size(plan, num_q_heads: int, num_kv_heads: int) -> int:
    a = _host_i32(plan) if not isinstance(plan, np.ndarray) else plan
    return _lib.check(lib().hpc_decode_workspace_size(_i32p(a), num_q_heads, num_kv_heads),
                      "hpc_decode_workspace_size")


def hpc_status_string(status: int) -> str:
    return lib().hpc_status_string(int(status)).decode()


# ----------------------------------------------------------- decode step ---

def _attn_args(q, k_cache, v_cache, block_table, seq_lens, plan_host, plan_dev, workspace, out, lse,
               num_kv_heads, sm_scale, k_scale, v_scale, tile_math="mfma"):
    if k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must have the same dtype")
    if q.dim() != 3 or k_cache.dim() != 4 or block_table.dim() != 2:
        raise ValueError("expected q [B,Hq,128], caches [pages,H_kv,64,128], block_table [B,max_pages]")
    params = make_params(q.shape[1], num_kv_heads, block_table.shape[1], k_cache.shape[0], k_cache.dtype,
                         sm_scale, k_scale, v_scale, head_dim=q.shape[2], page_size=k_cache.shape[2],
                         tile_math=tile_math)
    ph = plan_host if isinstance(plan_host, np.ndarray) else _host_i32(plan_host)
    if int(ph[1]) != q.shape[0] or block_table.shape[0] != q.shape[0] or seq_lens.shape[0] != q.shape[0]:
        raise ValueError("batch sizes of q, block_table, seq_lens and the plan differ")
    if k_cache.shape[1] != num_kv_heads or tuple(k_cache.shape) != tuple(v_cache.shape):
        raise ValueError("cache shapes disagree with num_kv_heads")
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != tuple(q.shape[:2]):
        raise ValueError("out must match q's shape and lse must be [B, Hq]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (ctypes.byref(params),
            _dev_ptr(q, "q", torch.bfloat16),
            _dev_ptr(k_cache, "k_cache", (torch.bfloat16, torch.float8_e4m3fn)),
            _dev_ptr(v_cache, "v_cache", (torch.bfloat16, torch.float8_e4m3fn)),
            _dev_ptr(block_table, "block_table", torch.int32),
            _dev_ptr(seq_lens, "seq_lens", torch.int32),
            _i32p(ph),
            _dev_ptr(plan_dev, "plan_dev", torch.int32),
            _dev_ptr(workspace, "workspace", allow_none=True),
            ctypes.c_int64(ws_bytes),
            _dev_ptr(out, "out", torch.bfloat16),
            _dev_ptr(lse, "lse", torch.float32))
    return args, ph


def hpc_decode_check(q, k_cache, v_cache, block_table, seq_lens, plan_host, plan_dev, workspace, out,
                     lse, *, num_kv_heads, sm_scale, k_scale=1.0, v_scale=1.0, tile_math="mfma") -> int:
    """Status that hpc_decode_attn would return for these arguments (no launch)."""
    args, _ = _attn_args(q, k_cache, v_cache, block_table, seq_lens, plan_host, plan_dev, workspace, out,
                         lse, num_kv_heads, sm_scale, k_scale, v_scale, tile_math)
    return lib().hpc_decode_check(*args)


def hpc_decode_attn(q, k_cache, v_cache, block_table, seq_lens, plan_host, plan_dev, workspace, out,
                    lse, *, num_kv_heads, sm_scale, k_scale=1.0, v_scale=1.0, stream=None,
                    tile_math="mfma") -> None:
    """One decode step on ``stream`` (default: torch's current stream); see hpc_decode.h."""
    args, _ = _attn_args(q, k_cache, v_cache, block_table, seq_lens, plan_host, plan_dev, workspace, out,
                         lse, num_kv_heads, sm_scale, k_scale, v_scale, tile_math)
    _lib.check(lib().hpc_decode_attn(*args, _stream_handle(stream)), "hpc_decode_attn")


class AttnLauncher:
    """A host-planned decode step for one prebuilt plan (``hpc_decode_attn``),
    with its arguments marshalled once.

    Calling it issues exactly one ``hpc_decode_attn`` on the stream given at
    construction (default: the current stream then).  The plan must already
    be on the device in ``plan_dev``; the plan words, the tensors and the
    workspace must stay alive and unchanged for the launcher's lifetime.
    """

    def __init__(self, q, k_cache, v_cache, block_table, seq_lens, plan_host, plan_dev, workspace, out, lse, *,
                 num_kv_heads, sm_scale, k_scale=1.0, v_scale=1.0, stream=None, tile_math="mfma"):
        args, ph = _attn_args(q, k_cache, v_cache, block_table, seq_lens, plan_host, plan_dev, workspace, out,
                              lse, num_kv_heads, sm_scale, k_scale, v_scale, tile_math)
        self._keep = (q, k_cache, v_cache, block_table, seq_lens, ph, plan_dev, workspace, out, lse)
        _lib.check(lib().hpc_decode_check(*args), "AttnLauncher")
        self._args = args + (_stream_handle(stream),)
        self._fn = lib().hpc_decode_attn

    def __call__(self) -> None:
        status = self._fn(*self._args)
        if status:
            _lib.check(status, "hpc_decode_attn")


# ------------------------------------------------ host-planned step in one call ---

def hpc_decode_plan_workspace_bound(batch: int, num_q_heads: int, num_kv_heads: int, n_workers: int) -> int:
    return _lib.check(lib().hpc_decode_plan_workspace_bound(batch, num_q_heads, num_kv_heads, n_workers),
                      "hpc_decode_plan_workspace_bound")


def hpc_decode_plan_attn(seq_lens_host, plan_host, plan_dev, q, k_cache, v_cache, block_table, seq_lens,
                         workspace, out, lse, *, num_kv_heads, n_workers, sm_scale, k_scale=1.0, v_scale=1.0,
                         stream=None, tile_math="mfma", entry_price=0) -> np.ndarray:
    """Plan the host lengths into ``plan_host`` (a host int32 buffer, pinned
    for an asynchronous upload), queue its copy to ``plan_dev`` and launch the
    step, in one native call; returns the plan words (a view of plan_host).
    The caller keeps plan_host unchanged until the copy has run on the stream."""
    lens = _host_i32(seq_lens_host).reshape(-1)
    params, args = _step_args(q, k_cache, v_cache, block_table, seq_lens, workspace, out, lse, num_kv_heads,
                              n_workers, sm_scale, k_scale, v_scale, tile_math, entry_price=entry_price)
    if lens.shape[0] != q.shape[0]:
        raise ValueError("seq_lens_host has the wrong batch size")
    ph = plan_host.numpy() if isinstance(plan_host, torch.Tensor) else plan_host
    if not isinstance(ph, np.ndarray) or ph.dtype != np.int32 or not ph.flags.c_contiguous:
        raise ValueError("plan_host must be a contiguous int32 host buffer")
    dev = _dev_ptr(plan_dev, "plan_dev", torch.int32)
    if plan_dev.numel() < ph.shape[0]:
        raise ValueError("plan_dev is smaller than plan_host")
    _lib.check(lib().hpc_decode_plan_attn(ctypes.byref(params), lens.ctypes.data, lens.shape[0], n_workers,
                                          ph.ctypes.data, ph.shape[0], dev, *args[2:], _stream_handle(stream)),
               "hpc_decode_plan_attn")
    return ph[:hpc_decode_plan_words(ph)]


class PlannedStepLauncher:
    """A host-planned decode step with its device arguments marshalled once.

    Each call plans the host lengths it is given into one of two pinned plan
    buffers, queues the plan's upload and launches the kernels, all in one
    ``hpc_decode_plan_attn`` call on the stream given at construction
    (default: the current stream then).  With ``in_place`` the kernels read
    the plan from the pinned buffer itself and no upload is queued.  An
    event recorded after each call guards its buffer: the call after next
    waits for it before rewriting the buffer.  Tensors must stay alive and
    unchanged in shape for the launcher's lifetime; ``plan_host`` is the last
    call's plan words.
    """

    def __init__(self, q, k_cache, v_cache, block_table, seq_lens, out, lse, *, num_kv_heads, n_workers,
                 sm_scale, k_scale=1.0, v_scale=1.0, workspace=None, stream=None, in_place=False,
                 tile_math="mfma", entry_price=0):
        B = q.shape[0]
        if workspace is None:
            need = hpc_decode_plan_workspace_bound(B, q.shape[1], num_kv_heads, n_workers)
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        self.params, args = _step_args(q, k_cache, v_cache, block_table, seq_lens, workspace, out, lse,
                                       num_kv_heads, n_workers, sm_scale, k_scale, v_scale, tile_math,
                                       entry_price=entry_price)
        self._keep = (q, k_cache, v_cache, block_table, seq_lens, out, lse, workspace)
        self.workspace = workspace
        self.batch, self.n_workers = int(B), int(n_workers)
        self._cap = hpc_decode_plan_size(B, num_kv_heads, n_workers)
        self._host = [torch.empty(self._cap, dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self._host_np = [h.numpy() for h in self._host]
        self.plan_dev = torch.empty(self._cap, dtype=torch.int32, device=q.device)
        self._stream = stream if stream is not None else torch.cuda.current_stream(q.device)
        self._events = [torch.cuda.Event(), torch.cuda.Event()]
        self._pending = [False, False]
        self._flip = 0
        self._last = None
        self._fn = lib().hpc_decode_plan_attn
        self._pre = (ctypes.byref(self.params),)
        self._post = args[2:] + (_stream_handle(self._stream),)
        self._host_ptr = [h.ctypes.data for h in self._host_np]
        self._dev_of = self._host_ptr if in_place else [self.plan_dev.data_ptr()] * 2

    def __call__(self, seq_lens_host) -> None:
        lens = seq_lens_host
        if not (type(lens) is np.ndarray and lens.dtype == np.int32 and lens.flags.c_contiguous
                and lens.shape == (self.batch,)):
            lens = _host_i32(lens).reshape(-1)
            if lens.shape[0] != self.batch:
                raise ValueError("seq_lens_host has the wrong batch size")
        i = self._flip
        self._flip = i ^ 1
        if self._pending[i]:
            self._events[i].synchronize()          # this buffer's last upload has run
        status = self._fn(*self._pre, lens.ctypes.data, self.batch, self.n_workers,
                          self._host_ptr[i], self._cap, self._dev_of[i], *self._post)
        if status:
            _lib.check(status, "hpc_decode_plan_attn")
        self._events[i].record(self._stream)
        self._pending[i] = True
        self._last = i

    @property
    def plan_host(self) -> np.ndarray:
        if self._last is None:
            raise RuntimeError("no step has been launched")
        h = self._host_np[self._last]
        return h[:hpc_decode_plan_words(h)]


# -------------------------------------------- device-scheduled decode step ---

def hpc_decode_step_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int, n_workers: int) -> int:
    return _lib.check(lib().hpc_decode_step_workspace_size(batch, num_q_heads, num_kv_heads, n_workers),
                      "hpc_decode_step_workspace_size")


def _step_args(q, k_cache, v_cache, block_table, seq_lens, workspace, out, lse, num_kv_heads, n_workers,
               sm_scale, k_scale, v_scale, tile_math="mfma", fused_merge=False, entry_price=0):
    if k_cache.dtype != v_cache.dtype or tuple(k_cache.shape) != tuple(v_cache.shape):
        raise ValueError("k_cache and v_cache must have the same dtype and shape")
    if q.dim() != 3 or k_cache.dim() != 4 or block_table.dim() != 2 or k_cache.shape[1] != num_kv_heads:
        raise ValueError("expected q [B,Hq,128], caches [pages,H_kv,64,128], block_table [B,max_pages]")
    B = q.shape[0]
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("batch sizes of q, block_table and seq_lens differ")
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != tuple(q.shape[:2]):
        raise ValueError("out must match q's shape and lse must be [B, Hq]")
    params = make_params(q.shape[1], num_kv_heads, block_table.shape[1], k_cache.shape[0], k_cache.dtype,
                         sm_scale, k_scale, v_scale, head_dim=q.shape[2], page_size=k_cache.shape[2],
                         tile_math=tile_math, fused_merge=fused_merge, entry_price=entry_price)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (params,
            (ctypes.c_int32(B), ctypes.c_int32(n_workers),
             _dev_ptr(q, "q", torch.bfloat16),
             _dev_ptr(k_cache, "k_cache", (torch.bfloat16, torch.float8_e4m3fn)),
             _dev_ptr(v_cache, "v_cache", (torch.bfloat16, torch.float8_e4m3fn)),
             _dev_ptr(block_table, "block_table", torch.int32),
             _dev_ptr(seq_lens, "seq_lens", torch.int32),
             _dev_ptr(workspace, "workspace", allow_none=True),
             ctypes.c_int64(ws_bytes),
             _dev_ptr(out, "out", torch.bfloat16),
             _dev_ptr(lse, "lse", torch.float32)))


def hpc_decode_step_check(q, k_cache, v_cache, block_table, seq_lens, workspace, out, lse, *, num_kv_heads,
                          n_workers, sm_scale, k_scale=1.0, v_scale=1.0, tile_math="mfma",
                          fused_merge=False, entry_price=0) -> int:
    params, args = _step_args(q, k_cache, v_cache, block_table, seq_lens, workspace, out, lse, num_kv_heads,
                              n_workers, sm_scale, k_scale, v_scale, tile_math, fused_merge, entry_price)
    return lib().hpc_decode_step_check(ctypes.byref(params), *args)


def hpc_decode_step(q, k_cache, v_cache, block_table, seq_lens, workspace, out, lse, *, num_kv_heads,
                    n_workers, sm_scale, k_scale=1.0, v_scale=1.0, stream=None, tile_math="mfma",
                    fused_merge=False, entry_price=0) -> None:
    """One decode step with the schedule derived on the device from ``seq_lens``.
    With ``fused_merge`` the decode kernel merges split sequences itself (no
    second kernel); the workspace must then be zero-filled before its first
    use, and every step leaves it so.  ``entry_price`` > 0 selects the
    priced partition (quarter tiles per unit start)."""
    params, args = _step_args(q, k_cache, v_cache, block_table, seq_lens, workspace, out, lse, num_kv_heads,
                              n_workers, sm_scale, k_scale, v_scale, tile_math, fused_merge, entry_price)
    _lib.check(lib().hpc_decode_step(ctypes.byref(params), *args, _stream_handle(stream)), "hpc_decode_step")


def hpc_decode_step_noalloc_max_bytes() -> int:
    return int(lib().hpc_decode_step_noalloc_max_bytes())


def hpc_decode_step_noalloc(q, k_cache, v_cache, block_table, seq_lens, out, lse, *, num_kv_heads, n_workers,
                            sm_scale, k_scale=1.0, v_scale=1.0, stream=None, tile_math="mfma",
                            entry_price=0) -> None:
    """hpc_decode_step with its scratch in the library's fixed per-GPU array
    (no workspace argument, no allocation); calls on one GPU share that array
    and must not overlap."""
    params, args = _step_args(q, k_cache, v_cache, block_table, seq_lens, None, out, lse, num_kv_heads,
                              n_workers, sm_scale, k_scale, v_scale, tile_math, False, entry_price)
    args = args[:7] + args[9:]       # no workspace pointer or size
    _lib.check(lib().hpc_decode_step_noalloc(ctypes.byref(params), *args, _stream_handle(stream)),
               "hpc_decode_step_noalloc")


def hpc_decode_plan_device(seq_lens: torch.Tensor, num_kv_heads: int, n_workers: int, max_pages_per_seq: int,
                           plan: torch.Tensor = None, stream=None, entry_price: int = 0) -> torch.Tensor:
    """The device-derived schedule as plan words (device int32 tensor, host-plan layout)."""
    B = int(seq_lens.shape[0])
    cap = hpc_decode_plan_size(B, num_kv_heads, n_workers)
    if plan is None:
        plan = torch.zeros(cap, dtype=torch.int32, device=seq_lens.device)
    _lib.check(lib().hpc_decode_plan_device(_dev_ptr(seq_lens, "seq_lens", torch.int32), B, num_kv_heads,
                                            n_workers, int(entry_price), max_pages_per_seq,
                                            _dev_ptr(plan, "plan", torch.int32),
                                            plan.numel(), _stream_handle(stream)), "hpc_decode_plan_device")
    return plan


class StepLauncher:
    """A device-scheduled decode step with its arguments marshalled once.


    Calling it issues exactly one ``hpc_decode_step`` on the stream given at
    construction (default: the current stream then); the tensors must stay
    alive and unchanged in shape for the launcher's lifetime.  Lengths are
    read from ``seq_lens`` on the device at every call.
    """

    def __init__(self, q, k_cache, v_cache, block_table, seq_lens, out, lse, *, num_kv_heads, n_workers,
                 sm_scale, k_scale=1.0, v_scale=1.0, workspace=None, stream=None, tile_math="mfma",
                 fused_merge=False, entry_price=0):
        need = hpc_decode_step_workspace_size(q.shape[0], q.shape[1], num_kv_heads, n_workers)
        if workspace is None:   # zero-filled, as the in-kernel merge needs
            workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=q.device)
        self._keep = (q, k_cache, v_cache, block_table, seq_lens, out, lse, workspace)
        self.params, args = _step_args(q, k_cache, v_cache, block_table, seq_lens, workspace, out, lse,
                                       num_kv_heads, n_workers, sm_scale, k_scale, v_scale, tile_math,
                                       fused_merge, entry_price)
        self.workspace = workspace
        self._args = (ctypes.byref(self.params),) + args + (_stream_handle(stream),)
        status = lib().hpc_decode_step_check(*self._args[:-1])
        _lib.check(status, "StepLauncher")
        self._fn = lib().hpc_decode_step

    def __call__(self) -> None:
        status = self._fn(*self._args)
        if status:
            _lib.check(status, "hpc_decode_step")


# ------------------------------------------------------------- profiling ---

def hpc_decode_profile_start(capacity: int) -> None:
    _lib.check(lib().hpc_decode_profile_start(capacity), "hpc_decode_profile_start")


def hpc_decode_profile_stop():
    """(summed decode-kernel ms, summed merge-kernel ms, calls recorded)."""
    d, c, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int32()
    _lib.check(lib().hpc_decode_profile_stop(ctypes.byref(d), ctypes.byref(c), ctypes.byref(n)),
               "hpc_decode_profile_stop")
    return d.value, c.value, n.value


def hpc_decode_trace_start(buffer: torch.Tensor) -> None:
    """Tracing window on: decode launches record 8 uint64 words per worker
    into ``buffer`` (device memory, >= 64 bytes per worker)."""
    _lib.check(lib().hpc_decode_trace_start(_dev_ptr(buffer, "buffer"), buffer.numel() * buffer.element_size()),
               "hpc_decode_trace_start")


def hpc_decode_trace_stop() -> None:
    _lib.check(lib().hpc_decode_trace_stop(), "hpc_decode_trace_stop")


def hpc_decode_wall_clock_hz() -> int:
    """Rate of the tracing stamps' clock (Hz) on the current device."""
    return _lib.check(lib().hpc_decode_wall_clock_hz(), "hpc_decode_wall_clock_hz")


def hpc_probe_read(buf: torch.Tensor, sink: torch.Tensor, n_workgroups: int, stream=None) -> None:
    nbytes = buf.numel() * buf.element_size()
    if sink.numel() < n_workgroups or sink.dtype != torch.float32:
        raise ValueError("sink must hold n_workgroups float32 values")
    _lib.check(lib().hpc_probe_read(_dev_ptr(buf, "buf"), nbytes, _dev_ptr(sink, "sink"), n_workgroups,
                                    _stream_handle(stream)), "hpc_probe_read")


def hpc_probe_read_timed(buf: torch.Tensor, sink: torch.Tensor, n_workgroups: int, stream=None) -> float:
    """One read-probe launch over `buf`; returns its dispatch-to-end duration in ms (synchronous)."""
    nbytes = buf.numel() * buf.element_size()
    if sink.numel() < n_workgroups or sink.dtype != torch.float32:
        raise ValueError("sink must hold n_workgroups float32 values")
    ms = ctypes.c_float()
    _lib.check(lib().hpc_probe_read_timed(_dev_ptr(buf, "buf"), nbytes, _dev_ptr(sink, "sink"), n_workgroups,
                                          _stream_handle(stream), ctypes.byref(ms)), "hpc_probe_read_timed")
    return ms.value


def hpc_probe_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst smaller than src")
    _lib.check(lib().hpc_probe_copy(_dev_ptr(src, "src"), _dev_ptr(dst, "dst"), nbytes,
                                    _stream_handle(stream)), "hpc_probe_copy")


# ------------------------------------------------------ per-step driver ---

class DecodeStep:
    """Buffers for repeated decode steps: plan, upload, attend.

    Holds two pinned host plan buffers (the host plans step n+1 while step
    n's upload may still be queued; an event guards reuse), one device plan
    buffer and a workspace that grows on demand.  All work is queued on one
    stream, so device buffers need no further synchronisation.
    """

    def __init__(self, num_q_heads: int, num_kv_heads: int, max_batch: int, n_workers: int,
                 device="cuda", stream=None, entry_price: int = 0):
        self.num_q_heads, self.num_kv_heads = int(num_q_heads), int(num_kv_heads)
        self.n_workers = int(n_workers)
        self.entry_price = int(entry_price)
        self.device = torch.device(device)
        self.stream = stream
        cap = hpc_decode_plan_size(max_batch, num_kv_heads, n_workers)
        self.max_batch = int(max_batch)
        self._host = [torch.empty(cap, dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self._host_ready = [None, None]
        self._flip = 0
        self.plan_dev = torch.empty(cap, dtype=torch.int32, device=self.device)
        self.workspace = torch.empty(0, dtype=torch.uint8, device=self.device)
        self.plan_host = None

    def _stream(self):
        return self.stream if self.stream is not None else torch.cuda.current_stream(self.device)

    def plan(self, seq_lens_host) -> np.ndarray:
        """Schedule this step's lengths and queue the plan's upload; returns the host plan."""
        lens = _host_i32(seq_lens_host).reshape(-1)
        if lens.shape[0] > self.max_batch:
            raise ValueError("batch larger than max_batch")
        i = self._flip
        self._flip ^= 1
        if self._host_ready[i] is not None:
            self._host_ready[i].synchronize()     # its previous upload has left the buffer
        words = hpc_decode_plan(lens, self.num_kv_heads, self.n_workers, out=self._host[i],
                                entry_price=self.entry_price)
        n = words.shape[0]
        s = self._stream()
        with torch.cuda.stream(s):
            self.plan_dev[:n].copy_(self._host[i][:n], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(s)
        self._host_ready[i] = ev
        need = hpc_decode_workspace_size(words, self.num_q_heads, self.num_kv_heads)
        if need > self.workspace.numel():
            self.workspace = torch.empty(max(need, 2 * self.workspace.numel()), dtype=torch.uint8,
                                         device=self.device)
        self.plan_host = words
        return words

    def attend(self, q, k_cache, v_cache, block_table, seq_lens_dev, out=None, lse=None, *,
               sm_scale, k_scale=1.0, v_scale=1.0, tile_math="mfma"):
        if self.plan_host is None:
            raise RuntimeError("call plan() before attend()")
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
        ws = self.workspace if self.workspace.numel() else None
        hpc_decode_attn(q, k_cache, v_cache, block_table, seq_lens_dev, self.plan_host, self.plan_dev, ws,
                        out, lse, num_kv_heads=self.num_kv_heads, sm_scale=sm_scale, k_scale=k_scale,
                        v_scale=v_scale, stream=self._stream(), tile_math=tile_math)
        return out, lse

    def __call__(self, seq_lens_host, q, k_cache, v_cache, block_table, seq_lens_dev, out=None, lse=None,
                 **scales):
        self.plan(seq_lens_host)
        return self.attend(q, k_cache, v_cache, block_table, seq_lens_dev, out, lse, **scales)
