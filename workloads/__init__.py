"""Seeded synthetic inputs for mixed-length paged GQA decode attention.

This module only draws inputs: sequence lengths, a shuffled block table, and
bf16 / fp8-e4m3 query and KV-cache values.  It holds none of the attention or
scheduling arithmetic, so both the float64 oracle (``oracle/``) and the HIP
path (``load_balanced_paged_step_amd``) can take their inputs from here
without sharing any code of the method.

The shapes follow the decode workloads on the pages ("vLLM x HPC-Ops:
High-Performance Attention and MoE Backends from Tencent Hunyuan",
§Attention Decode under Mixed-Length Batches: uniform 64x0.5K and the skewed
1x128K + 31x4K batch; §Attention Across Prefill, Extend and Decode Shapes:
the batch-8, 1K-KV decode shape) and the model head shape on the German
retelling (§Zwei neue HPC-Backends im vLLM-Ökosystem: 64 query heads, 8 KV
heads, head dim 128; one GPU of a TP8 deployment holds 8 query heads and one
KV head).  The FP8 cache flags (``--kv-cache-dtype fp8_e4m3 --block-size
64``) come from §Using HPC-Ops Backends in vLLM.

Recipe (fixed draw order, ``numpy.random.default_rng(seed)``):
  1. lengths (only for the log-uniform workload):
     ``L = clip(round(exp(U[ln 128, ln 65536])), 128, 65536)``;
  2. ``rng.permutation(N_pages)`` -> block table rows, in batch order;
  3. Q, then K, then V as N(0, 1) float32, cast to bf16 by torch (RNE);
     fp8 caches use ``scale = amax / 448`` per tensor, clamp to +-448, then
     torch's RNE cast to ``float8_e4m3fn``.
With ``poison=True`` one extra page (index ``N_pages``) is filled with NaN,
unused block-table slots point at it, and each sequence's last-page tail rows
are NaN too, so any read past a sequence's end shows up in the output.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

PAGE = 64          # tokens per KV page (= one scheduling tile)
HEAD_DIM = 128

BF16_NAN_BITS = 0x7FC0
E4M3_NAN_BITS = 0x7F
E4M3_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    """One decode workload: shapes only, no values."""
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    kv_dtype: str                      # "bf16" or "fp8_e4m3"
    seq_lens: tuple | None = None      # None -> drawn log-uniform from the seed
    loguniform: tuple = (128, 65536)
    description: str = ""


WORKLOADS = {
    1: Workload("tiny-4seq", 4, 8, 1, "bf16", (37, 64, 130, 200),
                description="batch 4, KV lengths 37/64/130/200, 8q/1kv, bf16"),
    2: Workload("uniform-64x512", 64, 8, 1, "bf16", (512,) * 64,
                description="batch 64, every KV length 512, 8q/1kv, bf16"),
    3: Workload("small-8x1024", 8, 8, 1, "bf16", (1024,) * 8,
                description="batch 8, every KV length 1024, 8q/1kv, bf16"),
    4: Workload("skewed-1x128k+31x4k", 32, 8, 1, "bf16", (131072,) + (4096,) * 31,
                description="batch 32 = one 131072-token sequence + 31 of 4096, 8q/1kv, bf16"),
    5: Workload("fp8-32xloguniform", 32, 64, 8, "fp8_e4m3", None,
                description="batch 32, KV lengths log-uniform in [128, 65536], 64q/8kv, fp8-e4m3 KV"),
}


@dataclass
class DecodeInputs:
    """Host-side (CPU) tensors for one decode step."""
    q: torch.Tensor            # bf16 [B, Hq, 128]
    k_cache: torch.Tensor      # bf16 or float8_e4m3fn [num_pages, H_kv, 64, 128]
    v_cache: torch.Tensor      # same
    block_table: torch.Tensor  # int32 [B, max_pages_per_seq]
    seq_lens: torch.Tensor     # int32 [B]
    num_q_heads: int
    num_kv_heads: int
    kv_dtype: str
    k_scale: float = 1.0
    v_scale: float = 1.0
    sm_scale: float = 1.0 / math.sqrt(HEAD_DIM)
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    def kv_bytes_attended(self) -> int:
        """KV bytes a decode step must read: valid tokens only."""
        per_tok = self.num_kv_heads * 2 * HEAD_DIM * self.k_cache.element_size()
        return int(self.seq_lens.to(torch.int64).sum()) * per_tok

    def algorithmic_bytes(self) -> int:
        """KV read + Q read + O written (bf16), per decode step."""
        qo = 2 * self.batch * self.num_q_heads * HEAD_DIM * 2
        return self.kv_bytes_attended() + qo

    # raw bit views for consumers that decode the formats themselves
    def q_bits(self) -> np.ndarray:
        return self.q.view(torch.int16).numpy().view(np.uint16)

    def k_bits(self) -> np.ndarray:
        return _cache_bits(self.k_cache)

    def v_bits(self) -> np.ndarray:
        return _cache_bits(self.v_cache)


def _cache_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    raise TypeError(f"unexpected cache dtype {t.dtype}")


def draw_loguniform_lengths(rng: np.random.Generator, batch: int, lo: int, hi: int) -> np.ndarray:
    x = np.exp(rng.uniform(math.log(lo), math.log(hi), size=batch))
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


def _normal_bf16(rng: np.random.Generator, shape) -> torch.Tensor:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16)


def _normal_fp8(rng: np.random.Generator, shape) -> tuple[torch.Tensor, float]:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    amax = float(np.abs(x).max()) if x.size else 1.0
    scale = amax / E4M3_MAX if amax > 0 else 1.0
    codes = torch.from_numpy(x).div_(scale).clamp_(-E4M3_MAX, E4M3_MAX)
    return codes.to(torch.float8_e4m3fn), scale


def make_inputs(seq_lens, num_q_heads: int, num_kv_heads: int, kv_dtype: str = "bf16",
                seed: int = 0, poison: bool = False, max_pages_per_seq: int | None = None,
                rng: np.random.Generator | None = None) -> DecodeInputs:
    """Draw one decode step's inputs for the given KV lengths.

    Pages hold all KV heads of 64 consecutive tokens of one sequence:
    ``cache[page, kv_head, row, dim]``; token t of sequence b lives in page
    ``block_table[b, t // 64]`` at row ``t % 64``.
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    lens = np.asarray(seq_lens, dtype=np.int64)
    B = int(lens.shape[0])
    n_pages_seq = (lens + PAGE - 1) // PAGE
    n_pages = int(n_pages_seq.sum())
    mpps = int(max(1, n_pages_seq.max() if B else 1)) if max_pages_per_seq is None else int(max_pages_per_seq)
    if B and n_pages_seq.max() > mpps:
        raise ValueError("max_pages_per_seq too small for the given lengths")

    perm = rng.permutation(n_pages).astype(np.int64)
    filler = max(n_pages, 1) if poison else 0
    bt = np.full((B, mpps), filler, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(n_pages_seq[b])
        bt[b, :n] = perm[off:off + n]
        off += n

    # an all-empty batch still gets one (never read) page so buffers are non-empty
    cache_shape = (max(n_pages, 1), num_kv_heads, PAGE, HEAD_DIM)
    q = _normal_bf16(rng, (B, num_q_heads, HEAD_DIM))
    if kv_dtype == "bf16":
        k = _normal_bf16(rng, cache_shape)
        v = _normal_bf16(rng, cache_shape)
        k_scale = v_scale = 1.0
    elif kv_dtype == "fp8_e4m3":
        k, k_scale = _normal_fp8(rng, cache_shape)
        v, v_scale = _normal_fp8(rng, cache_shape)
    else:
        raise ValueError(f"unknown kv dtype {kv_dtype!r}")

    if poison:   # values of the real pages do not depend on the poison flag
        k = torch.cat([k, torch.empty_like(k[:1])])
        v = torch.cat([v, torch.empty_like(v[:1])])
        _poison(k, bt, lens, k.shape[0] - 1)
        _poison(v, bt, lens, v.shape[0] - 1)

    return DecodeInputs(q=q, k_cache=k, v_cache=v, block_table=torch.from_numpy(bt),
                        seq_lens=torch.from_numpy(lens.astype(np.int32)),
                        num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, kv_dtype=kv_dtype,
                        k_scale=float(k_scale), v_scale=float(v_scale),
                        meta={"seed": seed, "poison": poison, "n_valid_pages": n_pages})


def _poison(cache: torch.Tensor, bt: np.ndarray, lens: np.ndarray, poison_page: int) -> None:
    if cache.dtype == torch.bfloat16:
        raw = cache.view(torch.int16)
        nan = np.int16(BF16_NAN_BITS)
    else:
        raw = cache.view(torch.uint8)
        nan = E4M3_NAN_BITS
    raw[poison_page].fill_(int(nan))
    for b, L in enumerate(lens.tolist()):
        if L % PAGE:
            last = int(bt[b, (L - 1) // PAGE])
            raw[last, :, L % PAGE:, :].fill_(int(nan))


def workload_lengths(cfg: int, seed: int | None = None) -> np.ndarray:
    """The sequence lengths of a named workload alone (the first draw of its
    generator, so they equal workload_inputs(cfg, seed).seq_lens)."""
    w = WORKLOADS[cfg]
    seed = cfg if seed is None else seed
    if w.seq_lens is None:
        return draw_loguniform_lengths(np.random.default_rng(seed), w.batch, *w.loguniform)
    return np.asarray(w.seq_lens, dtype=np.int64)


def workload_inputs(cfg: int, seed: int | None = None, poison: bool = False) -> DecodeInputs:
    """Inputs for one of the five named workloads (seed defaults to the workload number)."""
    w = WORKLOADS[cfg]
    seed = cfg if seed is None else seed
    rng = np.random.default_rng(seed)
    if w.seq_lens is None:
        lens = draw_loguniform_lengths(rng, w.batch, *w.loguniform)
    else:
        lens = np.asarray(w.seq_lens, dtype=np.int64)
    inp = make_inputs(lens, w.num_q_heads, w.num_kv_heads, w.kv_dtype, seed=seed,
                      poison=poison, rng=rng)
    inp.meta["workload"] = w.name
    return inp


# ---------------------------------------------------------------- prologue ---

@dataclass
class PrologueInputs:
    """One step's new token per sequence, before the fused prologue.

    ``cache`` holds the KV cache with room for the new token: its lengths are
    the cached lengths + 1, so the page of position ``positions[b]`` exists;
    the row of that position holds random (or poisoned) values until the
    prologue writes the new token there.  ``positions[b]`` = tokens cached
    before the step (the new token's position).
    """
    cache: DecodeInputs            # seq_lens = positions + 1 (the decode step after the prologue)
    positions: torch.Tensor        # int32 [B]
    q_in: torch.Tensor             # bf16 [B, Hq, 128]: the new token's query projection
    k_in: torch.Tensor             # bf16 [B, H_kv, 128]
    v_in: torch.Tensor             # bf16 [B, H_kv, 128]
    q_norm_w: torch.Tensor         # bf16 [128]
    k_norm_w: torch.Tensor         # bf16 [128]
    eps: float = 1e-6
    theta: float = 10000.0
    q_scale: float = 1.0 / 56.0    # fp8 query output: code = e4m3(q / q_scale)

    @staticmethod
    def bits(t: torch.Tensor) -> np.ndarray:
        return t.view(torch.int16).numpy().view(np.uint16)


def make_prologue_inputs(cached_lens, num_q_heads: int, num_kv_heads: int, kv_dtype: str = "bf16",
                         seed: int = 0, poison: bool = False, in_scale: float = 1.0) -> PrologueInputs:
    """Draw a prologue step: the cache (as ``make_inputs`` for cached_lens + 1,
    same rng), then Q, K, V of the new token as N(0, 1) * in_scale cast to
    bf16, then the two norm weights as N(1, 0.25^2) cast to bf16.  A negative
    cached length marks a padding slot: position -1, one cached token kept
    for the cache shape."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(cached_lens, dtype=np.int64)
    cache = make_inputs(np.where(lens < 0, 1, lens + 1), num_q_heads, num_kv_heads, kv_dtype, seed=seed,
                        poison=poison, rng=rng)
    B = int(lens.shape[0])

    def draw(shape, mean=0.0, sd=1.0):
        x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(sd) + np.float32(mean)
        return torch.from_numpy(x).to(torch.bfloat16)

    q_in = draw((B, num_q_heads, HEAD_DIM), sd=in_scale)
    k_in = draw((B, num_kv_heads, HEAD_DIM), sd=in_scale)
    v_in = draw((B, num_kv_heads, HEAD_DIM), sd=in_scale)
    q_w = draw((HEAD_DIM,), mean=1.0, sd=0.25)
    k_w = draw((HEAD_DIM,), mean=1.0, sd=0.25)
    return PrologueInputs(cache=cache, positions=torch.from_numpy(np.where(lens < 0, -1, lens).astype(np.int32)),
                          q_in=q_in, k_in=k_in, v_in=v_in, q_norm_w=q_w, k_norm_w=k_w)


# ----------------------------------------------------------------- prefill ---

@dataclass
class PrefillInputs:
    """A prefill / extend step: sequence b has ctx_b tokens cached before the
    step and n_b new tokens, whose K/V are already in the cache (lengths
    ctx_b + n_b); its queries are rows [q_start[b], q_start[b+1]) of q."""
    cache: DecodeInputs            # seq_lens = ctx + n (the cache the queries attend to)
    q: torch.Tensor                # bf16 [total, Hq, 128]
    q_start: torch.Tensor          # int32 [B + 1]

    @property
    def total(self) -> int:
        return int(self.q.shape[0])

    def q_bits(self) -> np.ndarray:
        return self.q.view(torch.int16).numpy().view(np.uint16)

    def q_lens(self) -> np.ndarray:
        s = self.q_start.numpy().astype(np.int64)
        return s[1:] - s[:-1]

    def flops(self) -> int:
        """4 * 128 FLOP (q.k and p.v) per (query head, visible token)."""
        lens = self.cache.seq_lens.numpy().astype(np.int64)
        n = self.q_lens()
        vis = sum(int(n_b * (L - n_b) + n_b * (n_b + 1) // 2) for n_b, L in zip(n, lens))
        return vis * self.cache.num_q_heads * 4 * HEAD_DIM


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    kv_dtype: str
    q_lens: tuple
    ctx_lens: tuple | None = None          # None -> log-uniform from the seed
    ctx_loguniform: tuple = (64, 16384)
    description: str = ""


PREFILL_WORKLOADS = {
    "prefill-q512": PrefillWorkload("prefill-q512", 64, 8, "bf16", (512,), (0,),
                                    description="one 512-token prompt, causal, 64q/8kv, bf16"),
    "prefill-q512-8q1kv": PrefillWorkload("prefill-q512-8q1kv", 8, 1, "bf16", (512,), (0,),
                                          description="one 512-token prompt, causal, 8q/1kv (one GPU of TP8)"),
    "extend-8x512": PrefillWorkload("extend-8x512", 64, 8, "bf16", (512,) * 8, None,
                                    description="8 chunks of 512 new tokens after log-uniform [64, 16384] "
                                                "cached tokens, 64q/8kv, bf16"),
    "extend-8x512-128q8kv": PrefillWorkload("extend-8x512-128q8kv", 128, 8, "bf16", (512,) * 8, None,
                                            description="extend-8x512 with 16 query heads per KV head, the "
                                                        "largest group the library takes (128q/8kv, bf16)"),
    "extend-8x256-fp8": PrefillWorkload("extend-8x256-fp8", 64, 8, "fp8_e4m3", (256,) * 8, None,
                                        description="8 chunks of 256 after log-uniform [64, 16384] cached "
                                                    "tokens, 64q/8kv, fp8-e4m3 KV"),
    "extend-32k+512-8q1kv": PrefillWorkload("extend-32k+512-8q1kv", 8, 1, "bf16", (512,), (32768,),
                                            description="one chunk of 512 new tokens after 32768 cached, 8q/1kv "
                                                        "(32 units of ~520 tiles each)"),
    "extend-128k+7x4k-8q1kv": PrefillWorkload("extend-128k+7x4k-8q1kv", 8, 1, "bf16", (512,) * 8,
                                              (131072,) + (4096,) * 7,
                                              description="8 chunks of 512, one after 131072 cached tokens and "
                                                          "seven after 4096, 8q/1kv (the skewed decode batch's "
                                                          "extend analogue)"),
}


def make_prefill_inputs(ctx_lens, q_lens, num_q_heads: int, num_kv_heads: int, kv_dtype: str = "bf16",
                        seed: int = 0, poison: bool = False, rng: np.random.Generator | None = None,
                        max_pages_per_seq: int | None = None) -> PrefillInputs:
    """Draw a prefill / extend step: the cache as ``make_inputs`` for
    ctx + n tokens (same rng), then the packed queries as N(0, 1) cast to
    bf16."""
    if rng is None:
        rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    n = np.asarray(q_lens, dtype=np.int64)
    cache = make_inputs(ctx + n, num_q_heads, num_kv_heads, kv_dtype, seed=seed, poison=poison, rng=rng,
                        max_pages_per_seq=max_pages_per_seq)
    q = _normal_bf16(rng, (int(n.sum()), num_q_heads, HEAD_DIM))
    q_start = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    return PrefillInputs(cache=cache, q=q, q_start=torch.from_numpy(q_start))


def prefill_workload_inputs(name: str, seed: int = 7, poison: bool = False) -> PrefillInputs:
    w = PREFILL_WORKLOADS[name]
    rng = np.random.default_rng(seed)
    if w.ctx_lens is None:
        ctx = draw_loguniform_lengths(rng, len(w.q_lens), *w.ctx_loguniform)
    else:
        ctx = np.asarray(w.ctx_lens, dtype=np.int64)
    inp = make_prefill_inputs(ctx, w.q_lens, w.num_q_heads, w.num_kv_heads, w.kv_dtype, seed=seed,
                              poison=poison, rng=rng)
    inp.cache.meta["workload"] = w.name
    return inp
