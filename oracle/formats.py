"""Bit-pattern decoders for the two KV-cache formats (float64 results).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the formats only: "native BF16 and FP8" (HPC-Ops blog,
§HPC-Ops: A Production Operator Library, Now in vLLM) and the KV-cache flag
``fp8_e4m3`` (§Using HPC-Ops Backends in vLLM).  The encodings used here are
the public definitions:

* bfloat16: the upper 16 bits of an IEEE-754 binary32.
* FP8 E4M3FN (OCP 8-bit floating point specification): 1 sign bit, 4
  exponent bits with bias 7, 3 mantissa bits; exponent 0 encodes subnormals
  ``m/8 * 2**-6``; there is no infinity; S.1111.111 is NaN; max 448.

Pinned by ``tests/test_oracle_formats.py`` against torch's casts for every
code.
"""

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3fn_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    exp = (b >> 3) & 0xF
    man = (b & 0x7).astype(np.float64)
    normal = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    subnormal = (man / 8.0) * 2.0 ** -6
    val = sign * np.where(exp == 0, subnormal, normal)
    return np.where((exp == 0xF) & ((b & 0x7) == 0x7), np.nan, val)


def cache_bits_to_f64(bits: np.ndarray, kv_format: str) -> np.ndarray:
    if kv_format == "bf16":
        return bf16_bits_to_f64(bits)
    if kv_format == "fp8_e4m3":
        return e4m3fn_bits_to_f64(bits)
    raise ValueError(f"unknown kv format {kv_format!r}")
