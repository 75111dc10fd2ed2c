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


# ---------------------------------------------------------------- encoders ---
# Rounding of a float64 value to the two formats, each taken once from the
# exact value (no intermediate float32), to nearest with ties to the even
# code, as both formats define it.

def _round_to_grid(a: np.ndarray, min_normal_exp: int, mant_bits: int) -> np.ndarray:
    """|a| (float64, finite, >= 0) rounded to nearest-even on the grid of a
    binary format with `mant_bits` stored mantissa bits whose smallest normal
    exponent is `min_normal_exp` (subnormals below it share that spacing)."""
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, min_normal_exp)
    # log2 can land one off near powers of two; fix e so that 2^e <= a < 2^(e+1)
    e = np.where((a >= np.exp2(e + 1)) & (a > 0), e + 1, e)
    e = np.where((a < np.exp2(e)) & (e > min_normal_exp), e - 1, e)
    spacing = np.exp2(e - mant_bits)
    return np.rint(a / spacing) * spacing          # np.rint rounds halves to even


def f64_to_bf16_bits(x) -> np.ndarray:
    """bfloat16 code of each value: nearest, ties to even; beyond the largest
    finite value (by at least half a step) -> infinity; NaN -> 0x7FC0."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    fin = np.isfinite(a)
    r = _round_to_grid(np.where(fin, a, 0.0), -126, 7)
    r = np.where(fin, r, np.inf)
    r = np.where(r > 3.3895313892515355e38, np.inf, r)     # above the largest finite bf16
    bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.signbit(x), bits | np.uint16(0x8000), bits)
    return np.where(np.isnan(x), np.uint16(0x7FC0), bits).astype(np.uint16)


E4M3_MAX = 448.0


def f64_to_e4m3fn_bits(x) -> np.ndarray:
    """OCP E4M3FN code of each value: nearest, ties to even, saturated to
    +-448 (the format has no infinity; a quantiser clamps to its largest
    value); the sign of a value that rounds to zero is kept; NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    a = np.where(np.isnan(x), 0.0, a)
    r = _round_to_grid(a, -6, 3)
    r = np.minimum(r, E4M3_MAX)
    # code from the value: exponent field and mantissa of r
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(r > 0, r, 1.0)))
    sub = r < 2.0 ** -6
    man_sub = np.rint(r / 2.0 ** -9)                              # 0..7 (8 = smallest normal)
    e = np.maximum(e, -6)
    man_norm = np.rint(r / np.exp2(e - 3)) - 8                      # 0..7
    code = np.where(sub, man_sub, (e + 7) * 8 + man_norm).astype(np.int64)
    code = np.where(np.signbit(x), code | 0x80, code)
    return np.where(np.isnan(x), 0x7F, code).astype(np.uint8)
