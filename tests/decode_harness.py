"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and the float64 oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import numpy as np
import torch
import xxhash

import load_balanced_paged_step_amd as hd
from oracle import decode_attention, cache_bits_to_f64

# max-abs output tolerance as a fraction of max|V| (V dequantised), per KV type
OUT_TOL = {"bf16": 1e-2, "fp8_e4m3": 3e-2}
# absolute log-sum-exp tolerance (natural log)
LSE_TOL = {"bf16": 1e-3, "fp8_e4m3": 1e-2}
# Per-unit output bound, for every (sequence, KV head) unit u and its G query
# heads: max|out_u - ref_u| <= UNIT_TOL * max|ref_u| + UNIT_ABS.  The output
# is an fp32 result rounded to bf16 (relative error <= 2^-8), and the
# probabilities are rounded to bf16 before P V (relative error <= 2^-8 each,
# summing like a random walk over the tokens, about 2^-8/sqrt(3) of |out| at
# the element that is largest), so the ratio stays near 4e-3 whatever the
# length; 1e-2 leaves a factor of about 2.5.  The same bound holds for fp8
# KV, whose codes widen to bf16 exactly.  The global bound above cannot see
# a long sequence's output at all: its |out| is far below 1e-2 max|V|.
UNIT_TOL = 1e-2
UNIT_ABS = 1e-6

# worst per-unit ratio max|out_u - ref_u| / max|ref_u| seen in this session,
# per KV type (printed in the test summary)
WORST_UNIT = {}


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)


def to_device(inp, device="cuda"):
    return dict(q=inp.q.to(device), k=inp.k_cache.to(device), v=inp.v_cache.to(device),
                bt=inp.block_table.to(device), sl=inp.seq_lens.to(device))


def run_hip(inp, n_workers: int, dev=None, return_step=False, tile_math="mfma"):
    """One decode step through DecodeStep (C++ planner, upload, HIP kernels)."""
    if dev is None:
        dev = to_device(inp)
    step = hd.DecodeStep(inp.num_q_heads, inp.num_kv_heads, inp.batch, n_workers)
    step.plan(inp.seq_lens)
    out, lse = step.attend(dev["q"], dev["k"], dev["v"], dev["bt"], dev["sl"], sm_scale=inp.sm_scale,
                           k_scale=inp.k_scale, v_scale=inp.v_scale, tile_math=tile_math)
    torch.cuda.synchronize()
    res = (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))
    return (res + (step,)) if return_step else res


# oracle results by a digest of everything they depend on: several tests run
# the oracle on the same seeded workload, and on the largest one it takes
# tens of seconds
_ORACLE_CACHE: dict = {}


def _inputs_digest(inp) -> tuple:
    h = xxhash.xxh3_128()
    for a in (inp.q_bits(), inp.k_bits(), inp.v_bits(), inp.block_table.numpy(), inp.seq_lens.numpy()):
        a = np.ascontiguousarray(a)
        h.update(str((a.dtype.str, a.shape)).encode())
        h.update(a.data)
    return (h.hexdigest(), inp.num_q_heads, inp.num_kv_heads, inp.kv_dtype, float(inp.sm_scale),
            float(inp.k_scale), float(inp.v_scale))


def run_oracle(inp):
    key = _inputs_digest(inp)
    hit = _ORACLE_CACHE.get(key)
    if hit is None:
        hit = decode_attention(inp.q_bits(), inp.k_bits(), inp.v_bits(), inp.block_table.numpy(),
                               inp.seq_lens.numpy(), num_q_heads=inp.num_q_heads,
                               num_kv_heads=inp.num_kv_heads, kv_format=inp.kv_dtype,
                               sm_scale=inp.sm_scale, k_scale=inp.k_scale, v_scale=inp.v_scale)
        if len(_ORACLE_CACHE) >= 16:
            _ORACLE_CACHE.pop(next(iter(_ORACLE_CACHE)))
        _ORACLE_CACHE[key] = hit
    return tuple(np.copy(x) for x in hit)


def max_abs_v(inp) -> float:
    """max |V| over the cache, dequantised: the maximum over the distinct
    codes the cache holds (one decode per distinct code, not per element)."""
    bits = np.ascontiguousarray(inp.v_bits()).reshape(-1)
    codes = np.flatnonzero(np.bincount(bits.view(np.uint8 if bits.itemsize == 1 else np.uint16)))
    v = cache_bits_to_f64(codes.astype(bits.dtype), inp.kv_dtype) * inp.v_scale
    v = v[np.isfinite(v)]
    return float(np.abs(v).max()) if v.size else 1.0


def compare(inp, got, ref, what=""):
    """Assert the HIP result is within tolerance of the oracle; returns error stats."""
    out, lse = got
    ref_out, ref_lse = ref
    tol = OUT_TOL[inp.kv_dtype] * max_abs_v(inp)
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = np.abs(out - ref_out)
    max_err = float(err.max()) if err.size else 0.0
    assert max_err <= tol, f"{what}: max|out-ref| = {max_err:.3e} > {tol:.3e}"
    neg = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), neg), f"{what}: -inf pattern of lse differs"
    lse_err = float(np.abs(lse[~neg] - ref_lse[~neg]).max()) if (~neg).any() else 0.0
    assert lse_err <= LSE_TOL[inp.kv_dtype], f"{what}: max|lse-ref| = {lse_err:.3e}"
    assert np.all(out[neg.nonzero()] == 0), f"{what}: empty sequences must give zeros"
    ratio, where = unit_check(out, ref_out, inp.num_kv_heads, what)
    prev = WORST_UNIT.get(inp.kv_dtype)
    if prev is None or ratio > prev[0]:
        WORST_UNIT[inp.kv_dtype] = (ratio, f"{what} {where}")
    return {"max_err": max_err, "tol": tol, "lse_err": lse_err, "worst_unit_ratio": ratio}


def unit_check(out, ref_out, num_kv_heads: int, what: str = ""):
    """Per-unit bound: for every (sequence b, KV head h) the G query heads'
    outputs satisfy max|out - ref| <= UNIT_TOL max|ref| + UNIT_ABS.  Returns
    the worst ratio max|out - ref| / max|ref| over non-zero units and where."""
    B, Hq = out.shape[:2]
    G = Hq // num_kv_heads
    o = out.reshape(B, num_kv_heads, G * out.shape[-1])
    r = ref_out.reshape(B, num_kv_heads, G * out.shape[-1])
    err = np.abs(o - r).max(axis=-1)
    mag = np.abs(r).max(axis=-1)
    bad = err > UNIT_TOL * mag + UNIT_ABS
    if bad.any():
        b, h = map(int, np.argwhere(bad)[0])
        raise AssertionError(f"{what}: unit (seq {b}, kv head {h}): max|out-ref| = {err[b, h]:.3e} > "
                             f"{UNIT_TOL:g} * max|ref| ({mag[b, h]:.3e}) + {UNIT_ABS:g}; "
                             f"{int(bad.sum())} units fail")
    nz = mag > 0
    if not nz.any():
        return 0.0, "(all units zero)"
    ratio = np.where(nz, err / np.where(nz, mag, 1.0), 0.0)
    b, h = map(int, np.unravel_index(np.argmax(ratio), ratio.shape))
    return float(ratio[b, h]), f"(seq {b}, kv head {h})"


def run_hip_plan(inp, plan_words, dev=None, tile_math="mfma"):
    """One decode step through hpc_decode_attn with a given host plan (any
    schedule in the plan word layout), uploaded once."""
    if dev is None:
        dev = to_device(inp)
    plan_host = np.ascontiguousarray(plan_words, dtype=np.int32)
    plan_dev = torch.from_numpy(plan_host).cuda()
    ws_bytes = hd.hpc_decode_workspace_size(plan_host, inp.num_q_heads, inp.num_kv_heads)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda") if ws_bytes > 0 else None
    out = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    hd.hpc_decode_attn(dev["q"], dev["k"], dev["v"], dev["bt"], dev["sl"], plan_host, plan_dev, ws, out, lse,
                       num_kv_heads=inp.num_kv_heads, sm_scale=inp.sm_scale, k_scale=inp.k_scale,
                       v_scale=inp.v_scale, tile_math=tile_math)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def run_hip_step(inp, n_workers: int, dev=None, tile_math="mfma", fused_merge=False, workspace=None,
                 entry_price=0):
    """One device-scheduled decode step (hpc_decode_step: schedule from the
    lengths on the GPU, decode and merge kernels, or the decode kernel alone
    with ``fused_merge``).  A given workspace is reused as it is."""
    if dev is None:
        dev = to_device(inp)
    ws_bytes = hd.hpc_decode_step_workspace_size(inp.batch, inp.num_q_heads, inp.num_kv_heads, n_workers)
    ws = workspace if workspace is not None else torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    hd.hpc_decode_step(dev["q"], dev["k"], dev["v"], dev["bt"], dev["sl"], ws, out, lse,
                       num_kv_heads=inp.num_kv_heads, n_workers=n_workers, sm_scale=inp.sm_scale,
                       k_scale=inp.k_scale, v_scale=inp.v_scale, tile_math=tile_math, fused_merge=fused_merge,
                       entry_price=entry_price)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
