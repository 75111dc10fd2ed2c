"""The device schedule's 32-bit quotient (quot_u32 in device_schedule.h),
modelled on the host at the extremes of its stated bounds.

The kernel takes floor(x / y) from a single-precision estimate: x and y
converted to float (round to nearest), the hardware reciprocal of y (within
one ulp of 1 / y), their product rounded to float, truncated to an integer,
clamped to qmax, then corrected by one step with 32-bit products.  The
schedule calls it with
  - range ends:  x = w rT < W^2, y = W <= 65536, qmax = W - 1;
  - first tile:  x = r < H n, y = n (tiles per sequence), qmax = H - 1,
                 H <= 4096 and H n <= T < 2^31.
Here the reciprocal is taken anywhere from two ulps below to two ulps above
the correctly rounded one.  The test checks that the estimate is within one
of the true quotient and that the correction makes it exact, including where
32-bit products would wrap without the clamp.
"""
import numpy as np
import pytest

U32 = 1 << 32


def _quot_u32_model(x, y, qmax, ulps):
    """Vectorised model of the kernel's steps for uint64 arrays x, y, qmax."""
    xf = x.astype(np.float32)
    rcp = (1.0 / y.astype(np.float64)).astype(np.float32)
    for _ in range(abs(ulps)):
        rcp = np.nextafter(rcp, np.float32(np.inf if ulps > 0 else 0), dtype=np.float32)
    est = np.floor((xf * rcp).astype(np.float32).astype(np.float64)).astype(np.uint64)
    q = np.minimum(est, qmax)
    p = (q * y) % U32                      # the kernel's 32-bit product
    assert np.all(q * y < U32), "a 32-bit product would wrap"
    down = p > x
    up = (~down) & (((x - p) % U32) >= y)
    q = np.where(down, q - 1, np.where(up, q + 1, q))
    return est, q


def _check(x, y, qmax):
    x, y, qmax = (np.asarray(v, dtype=np.uint64) for v in (x, y, qmax))
    true = x // y
    assert np.all(true <= qmax)
    for ulps in (-2, -1, 0, 1, 2):
        est, q = _quot_u32_model(x, y, qmax, ulps)
        lo = np.minimum(est, qmax)
        assert np.all(lo + 1 >= true) and np.all(lo <= true + 1), f"estimate off by more than one ({ulps} ulps)"
        np.testing.assert_array_equal(q, true)


def test_range_ends_at_the_largest_worker_counts():
    rng = np.random.default_rng(11)
    for W in (1, 2, 255, 256, 4097, 65535, 65536):
        w = np.concatenate([np.arange(0, min(W, 2048) + 1), rng.integers(0, W + 1, 4096), [W, W - 1]])
        rT = np.concatenate([rng.integers(0, W, w.size - 3), [W - 1, W - 1, 0]])
        _check(w * rT, np.full(w.size, W), np.full(w.size, W - 1))


def test_range_ends_match_the_exact_split():
    """equal_begin's sum w qT + quot(w rT, W) is floor(w T / W) for T < 2^31."""
    rng = np.random.default_rng(12)
    for W in (252, 256, 512, 65536):
        for T in (1, W - 1, W, 4032, 2**31 - 1, int(rng.integers(1, 2**31))):
            qT, rT = divmod(T, W)
            w = np.concatenate([np.arange(0, min(W, 1024) + 1), rng.integers(0, W + 1, 1024)]).astype(np.uint64)
            x = w * np.uint64(rT)
            _, q = _quot_u32_model(x, np.full(w.size, W, dtype=np.uint64), np.full(w.size, W - 1, dtype=np.uint64), 0)
            begin = w * np.uint64(qT) + q
            assert np.all(begin < U32)
            np.testing.assert_array_equal(begin, (w * np.uint64(T)) // np.uint64(W))


@pytest.mark.parametrize("H", [1, 2, 8, 64, 4096])
def test_first_tile_head_index(H):
    rng = np.random.default_rng(13 + H)
    n_max = (2**31 - 1) // H
    n = np.concatenate([rng.integers(1, n_max + 1, 3000), [1, 2, 63, 64, 65, n_max, n_max - 1]])
    r = (rng.random(n.size) * (H * n)).astype(np.uint64)
    r = np.minimum(r, np.uint64(H) * n.astype(np.uint64) - 1)
    # the last tile of each head and the first of the next, where rounding bites
    h = rng.integers(0, H, n.size).astype(np.uint64)
    edges = np.concatenate([h * n.astype(np.uint64) + n.astype(np.uint64) - 1, h * n.astype(np.uint64)])
    x = np.concatenate([r, edges])
    y = np.concatenate([n, n, n]).astype(np.uint64)
    _check(x, y, np.full(x.size, H - 1))
