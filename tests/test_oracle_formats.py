"""Pins for oracle.formats: every bf16 and E4M3FN code against torch's casts,
plus values fixed by the OCP FP8 specification."""
import numpy as np
import pytest
import torch

from oracle.formats import bf16_bits_to_f64, e4m3fn_bits_to_f64


def _same(a, b):
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


def test_bf16_all_codes_match_torch():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(bf16_bits_to_f64(codes), ref)


def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(e4m3fn_bits_to_f64(codes), ref)


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x38, 1.0), (0xB8, -1.0), (0x7E, 448.0), (0xFE, -448.0),
    (0x08, 2.0 ** -6), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x40, 2.0), (0x3C, 1.5),
])
def test_e4m3fn_spec_values(code, value):
    assert e4m3fn_bits_to_f64(np.array([code], dtype=np.uint8))[0] == value


def test_e4m3fn_nan_codes():
    v = e4m3fn_bits_to_f64(np.array([0x7F, 0xFF, 0x7E, 0x77], dtype=np.uint8))
    assert np.isnan(v[0]) and np.isnan(v[1]) and not np.isnan(v[2]) and v[3] == 240.0


def test_bf16_spec_values():
    v = bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x0001, 0x7F80, 0x3F81], dtype=np.uint16))
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 2.0 ** -133 and np.isinf(v[3])
    assert v[4] == 1.0 + 2.0 ** -7
