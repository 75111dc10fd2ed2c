"""Float64 CPU oracle for load-balanced paged GQA decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP
path never calls it, and it shares no code with the HIP path: it decodes the
bf16 / fp8-e4m3 bit patterns itself, gathers pages itself, and builds the
schedule itself.

Source pages: "vLLM x HPC-Ops: High-Performance Attention and MoE Backends
from Tencent Hunyuan" (English blog, and its Korean translation) and "vLLM
und Tencent Hunyuan streamen zwei HPC-Backends für NVIDIA-Hopper-GPUs
upstream" (German retelling).

Contents
  formats    bf16 and OCP FP8 E4M3FN bit patterns -> float64, and float64 ->
             codes (nearest, ties to even, rounded once)
  attention  paged decode attention as its plain definition (O1), attention
             over a token range plus the log-sum-exp merge (O2)
  plan       the per-step tile schedule (O3), an integer algorithm
  prefill    causal prefill / extend attention over the paged cache
  prologue   the step before attention: QK-norm, RoPE, paged append of the
             new token's K/V (fp8 quantised for an fp8 cache)

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against brute force, closed forms, invariants, or torch's own format casts.
"""

from .formats import (bf16_bits_to_f64, e4m3fn_bits_to_f64, cache_bits_to_f64, f64_to_bf16_bits,
                      f64_to_e4m3fn_bits)
from .attention import (decode_attention, range_attention, merge_partials,
                        split_decode_attention)
from .plan import build_plan, parse_plan, plan_size_words
from .prologue import decode_prologue, rms_norm, rope_angles, rope_rotate
from .prefill import prefill_attention

__all__ = [
    "bf16_bits_to_f64", "e4m3fn_bits_to_f64", "cache_bits_to_f64", "f64_to_bf16_bits", "f64_to_e4m3fn_bits",
    "decode_prologue", "rms_norm", "rope_angles", "rope_rotate", "prefill_attention",
    "decode_attention", "range_attention", "merge_partials", "split_decode_attention",
    "build_plan", "parse_plan", "plan_size_words",
]
