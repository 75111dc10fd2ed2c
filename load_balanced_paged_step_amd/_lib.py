"""ctypes declarations of ``libhpc_decode.so`` (the C ABI in include/*.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any step.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhpc_decode.so")

HPC_OK = 0
HPC_ERR_NULL = -1
HPC_ERR_INVALID = -2
HPC_ERR_UNSUPPORTED = -3
HPC_ERR_PLAN_MISMATCH = -4
HPC_ERR_TOO_SMALL = -5
HPC_ERR_HIP = -6

HPC_KV_BF16 = 0
HPC_KV_FP8_E4M3 = 1
HEAD_DIM = 128
PAGE = 64
MAX_GROUP = 16
HPC_TILE_MATH_MFMA = 0
HPC_TILE_MATH_VALU = 1
VALU_MAX_GROUP = 8
PLAN_HEADER_WORDS = 16


class hpc_decode_params(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("tile_math", ctypes.c_int32),
        ("fused_merge", ctypes.c_int32),
        ("entry_price", ctypes.c_int32),
    ]


class hpc_prologue_params(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("rope_theta", ctypes.c_float),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("q_scale", ctypes.c_float),
    ]


_I32P = ctypes.POINTER(ctypes.c_int32)
_F32P = ctypes.POINTER(ctypes.c_float)
_F64P = ctypes.POINTER(ctypes.c_double)
_VP = ctypes.c_void_p
_PP = ctypes.POINTER(hpc_decode_params)

# name -> (restype, argtypes)
SIGNATURES = {
    "hpc_decode_plan_size": (ctypes.c_int64, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    "hpc_decode_plan": (ctypes.c_int, [_I32P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _I32P,
                                       ctypes.c_int64]),
    "hpc_decode_plan_priced": (ctypes.c_int, [_I32P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                              _I32P, ctypes.c_int64]),
    "hpc_decode_plan_static_size": (ctypes.c_int64, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    "hpc_decode_plan_static": (ctypes.c_int, [_I32P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _I32P,
                                              ctypes.c_int64]),
    "hpc_decode_choose_workers": (ctypes.c_int32, [_I32P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.c_int32, ctypes.c_float]),
    "hpc_decode_pick_workers": (ctypes.c_int32, [_I32P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_int32]),
    "hpc_decode_pick_entry_price": (ctypes.c_int32, [_I32P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                     ctypes.c_int32]),
    "hpc_decode_pick_merge": (ctypes.c_int32, [_I32P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int32]),
    "hpc_decode_static_splits": (ctypes.c_int32, [_I32P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                  ctypes.c_int32]),
    "hpc_decode_plan_words": (ctypes.c_int64, [_I32P]),
    "hpc_decode_workspace_size": (ctypes.c_int64, [_I32P, ctypes.c_int32, ctypes.c_int32]),
    "hpc_decode_check": (ctypes.c_int, [_PP, _VP, _VP, _VP, _VP, _VP, _I32P, _VP, _VP, ctypes.c_int64,
                                        _VP, _VP]),
    "hpc_decode_attn": (ctypes.c_int, [_PP, _VP, _VP, _VP, _VP, _VP, _I32P, _VP, _VP, ctypes.c_int64,
                                       _VP, _VP, _VP]),
    "hpc_decode_plan_workspace_bound": (ctypes.c_int64, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                         ctypes.c_int32]),
    # host pointers as plain addresses: the per-step launcher passes integers
    "hpc_decode_plan_attn": (ctypes.c_int, [_PP, _VP, ctypes.c_int32, ctypes.c_int32, _VP, ctypes.c_int64, _VP,
                                            _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_int64, _VP, _VP, _VP]),
    "hpc_decode_step": (ctypes.c_int, [_PP, ctypes.c_int32, ctypes.c_int32, _VP, _VP, _VP, _VP, _VP, _VP,
                                       ctypes.c_int64, _VP, _VP, _VP]),
    "hpc_decode_step_noalloc": (ctypes.c_int, [_PP, ctypes.c_int32, ctypes.c_int32, _VP, _VP, _VP, _VP, _VP,
                                               _VP, _VP, _VP]),
    "hpc_decode_step_noalloc_max_bytes": (ctypes.c_int64, []),
    "hpc_decode_step_check": (ctypes.c_int, [_PP, ctypes.c_int32, ctypes.c_int32, _VP, _VP, _VP, _VP, _VP,
                                             _VP, ctypes.c_int64, _VP, _VP]),
    "hpc_decode_step_workspace_size": (ctypes.c_int64, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                        ctypes.c_int32]),
    "hpc_decode_plan_device": (ctypes.c_int, [_VP, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int32, _VP, ctypes.c_int64, _VP]),
    "hpc_decode_prologue": (ctypes.c_int, [ctypes.POINTER(hpc_prologue_params), ctypes.c_int32] + [_VP] * 12),
    "hpc_decode_prologue_check": (ctypes.c_int, [ctypes.POINTER(hpc_prologue_params), ctypes.c_int32]
                                  + [_VP] * 11),
    "hpc_prefill_units": (ctypes.c_int64, [_I32P, ctypes.c_int32, ctypes.c_int32]),
    "hpc_prefill_plan_size": (ctypes.c_int64, [_I32P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    "hpc_prefill_plan": (ctypes.c_int, [_I32P, _I32P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, _I32P, ctypes.c_int64, _I32P]),
    "hpc_prefill_workspace_size": (ctypes.c_int64, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    "hpc_prefill_attn": (ctypes.c_int, [_PP, ctypes.c_int32, ctypes.c_int32, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _VP, ctypes.c_int64, _VP, _VP,
                                        _VP]),
    "hpc_prefill_check": (ctypes.c_int, [_PP, ctypes.c_int32, ctypes.c_int32, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _VP, ctypes.c_int64, _VP,
                                         _VP]),
    "hpc_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "hpc_decode_trace_start": (ctypes.c_int, [_VP, ctypes.c_int64]),
    "hpc_decode_trace_stop": (ctypes.c_int, []),
    "hpc_decode_wall_clock_hz": (ctypes.c_int64, []),
    "hpc_decode_profile_start": (ctypes.c_int, [ctypes.c_int32]),
    "hpc_decode_profile_stop": (ctypes.c_int, [_F64P, _F64P, _I32P]),
    "hpc_probe_read": (ctypes.c_int, [_VP, ctypes.c_int64, _VP, ctypes.c_int32, _VP]),
    "hpc_probe_read_timed": (ctypes.c_int, [_VP, ctypes.c_int64, _VP, ctypes.c_int32, _VP,
                                            ctypes.POINTER(ctypes.c_float)]),
    "hpc_probe_copy": (ctypes.c_int, [_VP, _VP, ctypes.c_int64, _VP]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it is missing: build it first)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m load_balanced_paged_step_amd.build` "
                "(or __graft_entry__.build()) first")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class HpcDecodeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = int(status)
        msg = lib().hpc_status_string(int(status)).decode()
        super().__init__(f"{where}: {msg} (status {status})")


def check(status: int, where: str) -> int:
    if status < 0:
        raise HpcDecodeError(status, where)
    return status
