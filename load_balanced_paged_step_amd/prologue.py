"""Python binding of the fused decode prologue (``include/hpc_prologue.h``):
QK-norm, RoPE and the paged KV-cache append of each sequence's new token,
fp8-quantised for an fp8 cache, in one HIP kernel.

Argument marshalling only: every step runs in ``libhpc_decode.so``.
Method: "vLLM x HPC-Ops ...", §Attention Backend: Dynamic Load-Balanced
Scheduling (the fused attention prologue).
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import HEAD_DIM, PAGE, hpc_prologue_params, lib

__all__ = ["hpc_decode_prologue", "hpc_decode_prologue_check", "make_prologue_params", "PrologueLauncher"]


def _ptr(t, name, dtype, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (cuda) tensor")
    if t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def make_prologue_params(num_q_heads, num_kv_heads, max_pages_per_seq, num_pages, kv_dtype, *, eps, theta,
                         k_scale=1.0, v_scale=1.0, q_scale=1.0, head_dim=HEAD_DIM, page_size=PAGE):
    from . import kv_dtype_code
    code = kv_dtype if isinstance(kv_dtype, int) else kv_dtype_code(kv_dtype)
    return hpc_prologue_params(int(num_q_heads), int(num_kv_heads), int(head_dim), int(page_size),
                               int(max_pages_per_seq), int(num_pages), code, float(eps), float(theta),
                               float(k_scale), float(v_scale), float(q_scale))


def _args(q_in, k_in, v_in, q_norm_w, k_norm_w, positions, block_table, k_cache, v_cache, q_out, q_fp8,
          eps, theta, k_scale, v_scale, q_scale):
    if q_in.dim() != 3 or k_in.dim() != 3 or k_cache.dim() != 4 or block_table.dim() != 2:
        raise ValueError("expected q_in [B,Hq,128], k_in/v_in [B,H_kv,128], caches [pages,H_kv,64,128], "
                         "block_table [B,max_pages]")
    B, Hq, Hkv = q_in.shape[0], q_in.shape[1], k_in.shape[1]
    if (tuple(k_in.shape) != tuple(v_in.shape) or k_in.shape[0] != B or positions.shape[0] != B
            or block_table.shape[0] != B or tuple(q_out.shape) != tuple(q_in.shape)
            or (q_fp8 is not None and tuple(q_fp8.shape) != tuple(q_in.shape))
            or k_cache.shape[1] != Hkv or tuple(k_cache.shape) != tuple(v_cache.shape)
            or k_cache.dtype != v_cache.dtype or q_norm_w.numel() != q_in.shape[2]
            or k_norm_w.numel() != q_in.shape[2]):
        raise ValueError("prologue tensor shapes do not agree")
    params = make_prologue_params(Hq, Hkv, block_table.shape[1], k_cache.shape[0], k_cache.dtype, eps=eps,
                                  theta=theta, k_scale=k_scale, v_scale=v_scale, q_scale=q_scale,
                                  head_dim=q_in.shape[2], page_size=k_cache.shape[2])
    bf, f8 = torch.bfloat16, torch.float8_e4m3fn
    return params, [ctypes.c_int32(B), _ptr(q_in, "q_in", bf), _ptr(k_in, "k_in", bf), _ptr(v_in, "v_in", bf),
                    _ptr(q_norm_w, "q_norm_w", bf), _ptr(k_norm_w, "k_norm_w", bf),
                    _ptr(positions, "positions", torch.int32), _ptr(block_table, "block_table", torch.int32),
                    _ptr(k_cache, "k_cache", (bf, f8)), _ptr(v_cache, "v_cache", (bf, f8)),
                    _ptr(q_out, "q_out", bf), _ptr(q_fp8, "q_fp8", f8, allow_none=True)]


def hpc_decode_prologue_check(q_in, k_in, v_in, q_norm_w, k_norm_w, positions, block_table, k_cache, v_cache,
                              q_out, q_fp8=None, *, eps, theta, k_scale=1.0, v_scale=1.0, q_scale=1.0) -> int:
    params, args = _args(q_in, k_in, v_in, q_norm_w, k_norm_w, positions, block_table, k_cache, v_cache, q_out,
                         q_fp8, eps, theta, k_scale, v_scale, q_scale)
    return lib().hpc_decode_prologue_check(ctypes.byref(params), *args)


def hpc_decode_prologue(q_in, k_in, v_in, q_norm_w, k_norm_w, positions, block_table, k_cache, v_cache, q_out,
                        q_fp8=None, *, eps, theta, k_scale=1.0, v_scale=1.0, q_scale=1.0, stream=None) -> None:
    """One prologue step: q_out (and q_fp8) written, each sequence's new K/V
    appended to the caches at its position (see include/hpc_prologue.h)."""
    from . import _stream_handle
    params, args = _args(q_in, k_in, v_in, q_norm_w, k_norm_w, positions, block_table, k_cache, v_cache, q_out,
                         q_fp8, eps, theta, k_scale, v_scale, q_scale)
    _lib.check(lib().hpc_decode_prologue(ctypes.byref(params), *args, _stream_handle(stream)), "hpc_decode_prologue")


class PrologueLauncher:
    """hpc_decode_prologue with its arguments marshalled once: each call
    issues exactly one launch on the stream given at construction (default:
    the current stream then).  The tensors must stay alive and unchanged in
    shape; positions and caches are read on the device at every call."""

    def __init__(self, q_in, k_in, v_in, q_norm_w, k_norm_w, positions, block_table, k_cache, v_cache, q_out,
                 q_fp8=None, *, eps, theta, k_scale=1.0, v_scale=1.0, q_scale=1.0, stream=None):
        from . import _stream_handle
        self._keep = (q_in, k_in, v_in, q_norm_w, k_norm_w, positions, block_table, k_cache, v_cache, q_out, q_fp8)
        self.params, args = _args(q_in, k_in, v_in, q_norm_w, k_norm_w, positions, block_table, k_cache, v_cache,
                                  q_out, q_fp8, eps, theta, k_scale, v_scale, q_scale)
        self._args = (ctypes.byref(self.params), *args, _stream_handle(stream))
        _lib.check(lib().hpc_decode_prologue_check(*self._args[:-1]), "PrologueLauncher")
        self._fn = lib().hpc_decode_prologue

    def __call__(self) -> None:
        status = self._fn(*self._args)
        if status:
            _lib.check(status, "hpc_decode_prologue")
