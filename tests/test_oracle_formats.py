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


# ---- encoders: float64 -> code, nearest with ties to even --------------------

from oracle.formats import f64_to_bf16_bits, f64_to_e4m3fn_bits   # noqa: E402


def _finite_codes_bf16():
    c = np.arange(1 << 15, dtype=np.uint32).astype(np.uint16)      # non-negative codes
    v = bf16_bits_to_f64(c)
    return c[np.isfinite(v)], v[np.isfinite(v)]


def test_bf16_encoder_round_trips_every_code():
    c, v = _finite_codes_bf16()
    assert np.array_equal(f64_to_bf16_bits(v), c)
    assert np.array_equal(f64_to_bf16_bits(-v), c | np.uint16(0x8000))


def test_bf16_encoder_ties_go_to_the_even_code():
    c, v = _finite_codes_bf16()
    mid = (v[:-1] + v[1:]) / 2.0                  # exact in float64
    got = f64_to_bf16_bits(mid)
    even = np.where(c[:-1] % 2 == 0, c[:-1], c[1:])
    assert np.array_equal(got, even)
    # a hair either side of the midpoint goes to the nearer code
    up = np.nextafter(mid, np.inf)
    dn = np.nextafter(mid, -np.inf)
    assert np.array_equal(f64_to_bf16_bits(up), c[1:]) and np.array_equal(f64_to_bf16_bits(dn), c[:-1])


def test_bf16_encoder_matches_torch_on_random_values():
    # torch casts float64 to bfloat16 through float32, which rounds twice; on
    # float32-representable values the two agree
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-40, 38, 100000)).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f64_to_bf16_bits(x), ref)


def test_bf16_encoder_rounds_once():
    # 7935623376.008 lies 208 above the midpoint of bf16 codes 0x4FEC and
    # 0x4FED; rounding to float32 first would land on the midpoint and then
    # go to the even code 0x4FEC
    x = 7935623376.008081
    lo, hi = bf16_bits_to_f64(np.array([0x4FEC, 0x4FED], dtype=np.uint16))
    assert lo < (lo + hi) / 2 < x < hi and float(np.float32(x)) == (lo + hi) / 2
    assert f64_to_bf16_bits(np.array([x]))[0] == 0x4FED


def test_bf16_encoder_special_values():
    got = f64_to_bf16_bits(np.array([np.inf, -np.inf, np.nan, 3.4e38, -0.0, 2.0 ** -134]))
    assert got.tolist() == [0x7F80, 0xFF80, 0x7FC0, 0x7F80, 0x8000, 0x0000]


def _finite_codes_e4m3():
    c = np.arange(0x7F, dtype=np.uint8)          # 0 .. 0x7E: every non-negative finite code
    return c, e4m3fn_bits_to_f64(c)


def test_e4m3_encoder_round_trips_every_code():
    c, v = _finite_codes_e4m3()
    assert np.array_equal(f64_to_e4m3fn_bits(v), c)
    assert np.array_equal(f64_to_e4m3fn_bits(-v), c | 0x80)


def test_e4m3_encoder_ties_go_to_the_even_code():
    c, v = _finite_codes_e4m3()
    mid = (v[:-1] + v[1:]) / 2.0
    even = np.where(c[:-1] % 2 == 0, c[:-1], c[1:])
    assert np.array_equal(f64_to_e4m3fn_bits(mid), even)
    assert np.array_equal(f64_to_e4m3fn_bits(np.nextafter(mid, np.inf)), c[1:])
    assert np.array_equal(f64_to_e4m3fn_bits(np.nextafter(mid, -np.inf)), c[:-1])


def test_e4m3_encoder_saturates_and_keeps_signs():
    got = f64_to_e4m3fn_bits(np.array([449.0, 464.0, 479.9, 480.0, 1e9, -1e9, -0.0, -1e-9, 1e-9, np.nan]))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x80, 0x00, 0x7F]


def test_e4m3_encoder_matches_torch_within_range():
    rng = np.random.default_rng(1)
    x = np.concatenate([np.clip(rng.standard_normal(100000) * 60, -448, 448), rng.standard_normal(50000) * 0.01])
    x = x.astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(f64_to_e4m3fn_bits(x), ref)
