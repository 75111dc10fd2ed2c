"""C-ABI tests that need no GPU: the library loads, exports every declared
symbol, its C++ planner equals the oracle's schedule word for word, and every
host-checkable error is reported before anything is launched."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import load_balanced_paged_step_amd as hd
from load_balanced_paged_step_amd import _lib
from oracle.plan import build_plan, build_static_plan, plan_size_words, static_split_count

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(hpc_[A-Za-z0-9_]+)\s*\(",
                             text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert "hpc_decode_plan" in names and "hpc_decode_attn" in names and len(names) >= 10
    lib = _lib.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"{n} has no ctypes signature"


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert hd.hpc_status_string(code) != "unknown status"
    assert hd.hpc_status_string(-99) == "unknown status"


def _cpp_plan(lens, H, W):
    return hd.hpc_decode_plan(np.asarray(lens, dtype=np.int32), H, W)


@pytest.mark.parametrize("lens,H,W", [
    ([37, 64, 130, 200], 1, 4), ([0, 100, 10], 2, 4), ([65], 1, 5), ([1, 0, 128], 1, 1),
    ([131072] + [4096] * 31, 1, 256), ([131072] + [4096] * 31, 1, 1024), ([512] * 64, 1, 256),
    ([1024] * 8, 1, 256), ([0, 0, 0], 8, 7), ([5000] * 3, 8, 700),
])
def test_cpp_plan_equals_oracle(lens, H, W):
    got = _cpp_plan(lens, H, W)
    ref = build_plan(lens, H, W)
    assert got.dtype == np.int32 and np.array_equal(got, ref)
    assert hd.hpc_decode_plan_size(len(lens), H, W) == plan_size_words(len(lens), H, W)


def test_cpp_plan_exhaustive_small():
    for L in range(0, 131):
        for H in (1, 2):
            for W in range(1, 10):
                assert np.array_equal(_cpp_plan([L], H, W), build_plan([L], H, W))
    vals = [0, 1, 63, 64, 65, 128, 129]
    for a in vals:
        for b in vals:
            for W in (1, 2, 3, 5, 8):
                assert np.array_equal(_cpp_plan([a, b], 2, W), build_plan([a, b], 2, W))


@settings(max_examples=300, deadline=None)
@given(lens=st.lists(st.integers(0, 70000), min_size=0, max_size=48), H=st.integers(1, 8),
       W=st.integers(1, 1500))
def test_cpp_plan_random(lens, H, W):
    assert np.array_equal(_cpp_plan(lens, H, W), build_plan(lens, H, W))


PRICES = (1, 2, 4, 8, 16, 64)


@pytest.mark.parametrize("c", PRICES)
@pytest.mark.parametrize("lens,H,W", [
    ([37, 64, 130, 200], 1, 4), ([0, 100, 10], 2, 4), ([64, 64, 64, 640], 1, 2), ([64, 0, 192], 2, 2),
    ([131072] + [4096] * 31, 1, 252), ([131072] + [4096] * 31, 1, 256), ([512] * 64, 1, 256),
    ([0, 0, 0], 8, 7), ([5000] * 3, 8, 700),
])
def test_cpp_priced_plan_equals_oracle(lens, H, W, c):
    got = hd.hpc_decode_plan(np.asarray(lens, dtype=np.int32), H, W, entry_price=c)
    assert np.array_equal(got, build_plan(lens, H, W, c))


def test_cpp_priced_plan_cost_limit():
    """16 units of 2^25 - 1 tiles: C = 4 T + 16 c = 2^31 - 64 + 16 c, priced
    only while below 2^31 (c <= 3).  Each worker's share then starts where
    the cost prefix says (units of equal cost: worker w of 64 at unit w / 4)."""
    lens = np.array([64 * (2 ** 25 - 1)], dtype=np.int32)
    for c, applied in ((2, 2), (3, 3), (4, 0), (16, 0)):
        words = hd.hpc_decode_plan(lens, 16, 64, entry_price=c)
        assert int(words[9]) == applied
        wp = words[16:16 + 65]
        ents = words[16 + 65:16 + 65 + 4 * int(words[5])].reshape(-1, 4)
        starts = [tuple(ents[wp[w]][:2]) for w in range(0, 64, 4)]
        assert starts == [(w // 4, 0) for w in range(0, 64, 4)]


@settings(max_examples=300, deadline=None)
@given(lens=st.lists(st.integers(0, 70000), min_size=0, max_size=48), H=st.integers(1, 8),
       W=st.integers(1, 1500), c=st.sampled_from(PRICES))
def test_cpp_priced_plan_random(lens, H, W, c):
    got = hd.hpc_decode_plan(np.asarray(lens, dtype=np.int32), H, W, entry_price=c)
    assert np.array_equal(got, build_plan(lens, H, W, c))


def test_priced_plan_errors():
    lib = _lib.lib()
    lens = np.array([100, 200], dtype=np.int32)
    p = lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    buf = np.zeros(hd.hpc_decode_plan_size(2, 1, 4), dtype=np.int32)
    q = buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert lib.hpc_decode_plan_priced(p, 2, 1, 4, 0, q, buf.size) == hd.HPC_OK
    assert lib.hpc_decode_plan_priced(p, 2, 1, 4, hd.MAX_ENTRY_PRICE, q, buf.size) == hd.HPC_OK
    assert lib.hpc_decode_plan_priced(p, 2, 1, 4, -1, q, buf.size) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_plan_priced(p, 2, 1, 4, hd.MAX_ENTRY_PRICE + 1, q, buf.size) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_plan_priced(None, 2, 1, 4, 4, q, buf.size) == hd.HPC_ERR_NULL
    assert lib.hpc_decode_plan_priced(p, 2, 1, 4, 4, q, 3) == hd.HPC_ERR_TOO_SMALL


@pytest.mark.parametrize("lens,H,S", [
    ([37, 64, 130, 200], 1, 2), ([0, 320], 2, 3), ([130], 1, 4), ([0, 0], 1, 8), ([1, 0, 128], 1, 1),
    ([131072] + [4096] * 31, 1, 8), ([131072] + [4096] * 31, 1, 128), ([512] * 64, 1, 4), ([5000] * 3, 8, 7),
])
def test_cpp_static_plan_equals_oracle(lens, H, S):
    got = hd.hpc_decode_plan_static(np.asarray(lens, dtype=np.int32), H, S)
    assert np.array_equal(got, build_static_plan(lens, H, S))
    assert hd.hpc_decode_plan_static_size(len(lens), H, S) >= got.shape[0]


@settings(max_examples=200, deadline=None)
@given(lens=st.lists(st.integers(0, 70000), min_size=0, max_size=40), H=st.integers(1, 8),
       S=st.integers(1, 200))
def test_cpp_static_plan_random(lens, H, S):
    got = hd.hpc_decode_plan_static(np.asarray(lens, dtype=np.int32), H, S)
    assert np.array_equal(got, build_static_plan(lens, H, S))


@settings(max_examples=200, deadline=None)
@given(lens=st.lists(st.integers(0, 300000), min_size=0, max_size=64), H=st.integers(1, 8),
       cus=st.integers(1, 1024), cap=st.integers(1, 256))
def test_cpp_static_splits_equal_oracle(lens, H, cus, cap):
    assert hd.hpc_decode_static_splits(np.asarray(lens, dtype=np.int32), H, cus, cap) == \
        static_split_count(lens, H, cus, cap)


def test_static_plan_errors():
    lib = hd.lib()
    buf = np.zeros(64, dtype=np.int32)
    lens = np.asarray([100, 200], dtype=np.int32)
    i32p = ctypes.POINTER(ctypes.c_int32)
    assert lib.hpc_decode_plan_static(lens.ctypes.data_as(i32p), 2, 1, 0, buf.ctypes.data_as(i32p), 64) == _lib.HPC_ERR_INVALID
    assert lib.hpc_decode_plan_static(lens.ctypes.data_as(i32p), 2, 0, 2, buf.ctypes.data_as(i32p), 64) == _lib.HPC_ERR_INVALID
    assert lib.hpc_decode_plan_static(None, 2, 1, 2, buf.ctypes.data_as(i32p), 64) == _lib.HPC_ERR_NULL
    assert lib.hpc_decode_plan_static(lens.ctypes.data_as(i32p), 2, 1, 2, buf.ctypes.data_as(i32p), 8) == _lib.HPC_ERR_TOO_SMALL
    bad = np.asarray([100, -1], dtype=np.int32)
    assert lib.hpc_decode_plan_static(bad.ctypes.data_as(i32p), 2, 1, 2, buf.ctypes.data_as(i32p), 64) == _lib.HPC_ERR_INVALID
    assert lib.hpc_decode_plan_static_size(-1, 1, 1) == _lib.HPC_ERR_INVALID
    assert lib.hpc_decode_plan_static_size(1, 1, 0) == _lib.HPC_ERR_INVALID


def test_workspace_size():
    plan = _cpp_plan([131072] + [4096] * 31, 1, 256)
    P = int(plan[6])
    o = P * 8 * 128 * 4
    assert hd.hpc_decode_workspace_size(plan, 8, 1) == (o + 255) // 256 * 256 + P * 8 * 4
    assert hd.hpc_decode_workspace_size(_cpp_plan([64], 1, 1), 8, 1) == 0


def test_plan_errors():
    lib = _lib.lib()
    buf = np.zeros(1000, dtype=np.int32)
    lens = np.array([10, 20], dtype=np.int32)
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert lib.hpc_decode_plan(p(lens), 2, 1, 0, p(buf), 1000) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_plan(p(lens), 2, 0, 4, p(buf), 1000) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_plan(p(lens), -1, 1, 4, p(buf), 1000) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_plan(None, 2, 1, 4, p(buf), 1000) == hd.HPC_ERR_NULL
    assert lib.hpc_decode_plan(p(lens), 2, 1, 4, None, 1000) == hd.HPC_ERR_NULL
    assert lib.hpc_decode_plan(p(lens), 2, 1, 4, p(buf), 10) == hd.HPC_ERR_TOO_SMALL
    neg = np.array([10, -1], dtype=np.int32)
    assert lib.hpc_decode_plan(p(neg), 2, 1, 4, p(buf), 1000) == hd.HPC_ERR_INVALID
    huge = np.full(40000, 2 ** 31 - 1, dtype=np.int32)        # T >= 2^31 tiles
    big = np.zeros(hd.hpc_decode_plan_size(40000, 1, 4), dtype=np.int32)
    assert lib.hpc_decode_plan(p(huge), 40000, 1, 4, p(big), big.shape[0]) == hd.HPC_ERR_INVALID
    with pytest.raises(hd.HpcDecodeError):
        hd.hpc_decode_plan([1, 2], 1, 0)
    assert lib.hpc_decode_plan_size(-1, 1, 1) < 0 and lib.hpc_decode_plan_size(1, 1, 0) < 0


class _Fake:
    """Host-side stand-ins for device buffers: hpc_decode_check never dereferences them."""

    def __init__(self, lens=(37, 200), H=1, Hq=8, W=4):
        self.lens = np.asarray(lens, dtype=np.int32)
        self.plan = _cpp_plan(self.lens, H, W).copy()
        self.params = hd.make_params(Hq, H, 4, 8, hd.HPC_KV_BF16, 1 / np.sqrt(128))
        self.ws = hd.hpc_decode_workspace_size(self.plan, Hq, H)
        self.ptr = ctypes.c_void_p(0x1000)

    def check(self, **over):
        lib = _lib.lib()
        a = dict(p=ctypes.byref(self.params), q=self.ptr, k=self.ptr, v=self.ptr, bt=self.ptr,
                 sl=self.ptr, ph=self.plan.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                 pd=self.ptr, ws=self.ptr, wsb=self.ws, out=self.ptr, lse=self.ptr)
        a.update(over)
        return lib.hpc_decode_check(a["p"], a["q"], a["k"], a["v"], a["bt"], a["sl"], a["ph"], a["pd"],
                                    a["ws"], a["wsb"], a["out"], a["lse"])


def test_check_accepts_a_consistent_call():
    assert _Fake().check() == hd.HPC_OK


@pytest.mark.parametrize("field", ["q", "k", "v", "bt", "sl", "ph", "pd", "out", "lse", "p"])
def test_check_null_pointers(field):
    assert _Fake().check(**{field: None}) == hd.HPC_ERR_NULL


def test_check_null_workspace_only_when_needed():
    f = _Fake()
    assert f.ws > 0 and f.check(ws=None) == hd.HPC_ERR_NULL
    g = _Fake(lens=(64,), W=1)
    assert g.ws == 0 and g.check(ws=None, wsb=0) == hd.HPC_OK


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 64, hd.HPC_ERR_UNSUPPORTED), ("page_size", 16, hd.HPC_ERR_UNSUPPORTED),
    ("kv_dtype", 7, hd.HPC_ERR_UNSUPPORTED),
    ("num_q_heads", 0, hd.HPC_ERR_INVALID), ("num_kv_heads", 0, hd.HPC_ERR_INVALID),
    ("max_pages_per_seq", 0, hd.HPC_ERR_INVALID), ("num_pages", 0, hd.HPC_ERR_INVALID),
    ("sm_scale", float("nan"), hd.HPC_ERR_INVALID), ("v_scale", float("inf"), hd.HPC_ERR_INVALID),
    ("entry_price", -1, hd.HPC_ERR_INVALID), ("entry_price", hd.MAX_ENTRY_PRICE + 1, hd.HPC_ERR_INVALID),
])
def test_check_bad_params(field, value, code):
    f = _Fake()
    setattr(f.params, field, value)
    assert f.check() == code


def test_check_heads_not_a_multiple():
    f = _Fake(H=2, Hq=16)
    f.params.num_q_heads = 9
    assert f.check() == hd.HPC_ERR_INVALID


def test_check_group_too_large():
    f = _Fake(Hq=32)
    assert f.check() == hd.HPC_ERR_UNSUPPORTED


def test_check_tile_math():
    f = _Fake(H=2, Hq=16)                      # G = 8: both tile maths
    for code in (hd.HPC_TILE_MATH_MFMA, hd.HPC_TILE_MATH_VALU):
        f.params.tile_math = code
        assert f.check() == hd.HPC_OK
    for bad in (2, -1):
        f.params.tile_math = bad
        assert f.check() == hd.HPC_ERR_INVALID
    g = _Fake(H=1, Hq=16)                      # G = 16: MFMA only
    assert g.check() == hd.HPC_OK
    g.params.tile_math = hd.HPC_TILE_MATH_VALU
    assert g.check() == hd.HPC_ERR_UNSUPPORTED
    assert hd.make_params(8, 1, 4, 8, hd.HPC_KV_BF16, 0.1, tile_math="valu").tile_math == hd.HPC_TILE_MATH_VALU
    assert hd.make_params(8, 1, 4, 8, hd.HPC_KV_BF16, 0.1).tile_math == hd.HPC_TILE_MATH_MFMA
    with pytest.raises(ValueError):
        hd.make_params(8, 1, 4, 8, hd.HPC_KV_BF16, 0.1, tile_math="simd")


def test_check_fused_merge():
    f = _Fake()
    f.params.fused_merge = 1                   # the host-planned step has no in-kernel merge
    assert f.check() == hd.HPC_ERR_UNSUPPORTED
    f.params.fused_merge = 2
    assert f.check() == hd.HPC_ERR_INVALID
    lib = _lib.lib()
    ptr = ctypes.c_void_p(0x1000)
    need = hd.hpc_decode_step_workspace_size(2, 8, 1, 16)
    for val, code in ((0, hd.HPC_OK), (1, hd.HPC_OK), (-1, hd.HPC_ERR_INVALID), (3, hd.HPC_ERR_INVALID)):
        params = hd.make_params(8, 1, 4, 8, hd.HPC_KV_BF16, 1 / np.sqrt(128))
        params.fused_merge = val
        assert lib.hpc_decode_step_check(ctypes.byref(params), 2, 16, ptr, ptr, ptr, ptr, ptr, ptr, need,
                                         ptr, ptr) == code, val


def test_params_struct_matches_header():
    """The ctypes mirror of hpc_decode_params has the header's fields, in order."""
    import re
    hdr = open(os.path.join(ROOT, "include", "hpc_decode.h")).read()
    body = re.search(r"typedef struct hpc_decode_params \{(.*?)\} hpc_decode_params;", hdr, re.S).group(1)
    fields = re.findall(r"^\s*(?:int32_t|float)\s+(\w+);", body, re.M)
    assert fields == [f[0] for f in hd.hpc_decode_params._fields_]
    assert ctypes.sizeof(hd.hpc_decode_params) == 4 * len(fields)


def test_check_plan_mismatches():
    f = _Fake()
    assert f.check(wsb=f.ws - 1) == hd.HPC_ERR_TOO_SMALL
    f.params.max_pages_per_seq = 3            # the 200-token sequence needs 4 pages
    assert f.check() == hd.HPC_ERR_INVALID
    g = _Fake(H=2, Hq=16)
    g.params.num_kv_heads = 1
    g.params.num_q_heads = 8
    assert g.check() == hd.HPC_ERR_PLAN_MISMATCH
    for word, bad in [(0, 2), (8, 32), (16, 1)]:
        h = _Fake()
        h.plan[word] = bad
        assert h.check() == hd.HPC_ERR_PLAN_MISMATCH
    k = _Fake()
    e0 = 16 + int(k.plan[3]) + 1
    k.plan[e0 + 2] = k.plan[e0 + 1]            # empty tile range
    assert k.check() == hd.HPC_ERR_PLAN_MISMATCH
    m = _Fake()
    m.plan[e0 + 3] = int(m.plan[6])            # slot beyond n_partials
    assert m.check() == hd.HPC_ERR_PLAN_MISMATCH


def test_step_check_errors():
    lib = _lib.lib()
    ptr = ctypes.c_void_p(0x1000)
    params = hd.make_params(8, 1, 4, 8, hd.HPC_KV_BF16, 1 / np.sqrt(128))
    need = hd.hpc_decode_step_workspace_size(2, 8, 1, 16)
    P = 2 * 16            # two partial slots per worker
    al = lambda x: (x + 255) // 256 * 256
    assert need == al(al(P * 8 * 128 * 4) + P * 8 * 4) + 6 * 2 * 4

    def chk(batch=2, W=16, ws=ptr, wsb=need, **over):
        a = dict(q=ptr, k=ptr, v=ptr, bt=ptr, sl=ptr, out=ptr, lse=ptr)
        a.update(over)
        return lib.hpc_decode_step_check(ctypes.byref(params), batch, W, a["q"], a["k"], a["v"], a["bt"],
                                         a["sl"], ws, wsb, a["out"], a["lse"])
    assert chk() == hd.HPC_OK
    assert chk(sl=None) == hd.HPC_ERR_NULL and chk(ws=None) == hd.HPC_ERR_NULL
    assert chk(wsb=need - 1) == hd.HPC_ERR_TOO_SMALL
    assert chk(batch=0) == hd.HPC_ERR_INVALID and chk(W=0) == hd.HPC_ERR_INVALID
    assert chk(batch=5000, wsb=1 << 40) == hd.HPC_ERR_UNSUPPORTED
    assert chk(W=65537, wsb=1 << 40) == hd.HPC_ERR_UNSUPPORTED
    for price, code in ((hd.MAX_ENTRY_PRICE, hd.HPC_OK), (hd.MAX_ENTRY_PRICE + 1, hd.HPC_ERR_INVALID),
                        (-1, hd.HPC_ERR_INVALID)):
        params.entry_price = price
        assert chk() == code
    params.entry_price = 0
    params.max_pages_per_seq = 1 << 20
    assert chk(batch=2048, wsb=1 << 40) == hd.HPC_ERR_INVALID       # tile indices beyond int32
    params.max_pages_per_seq = 4
    params.head_dim = 64
    assert chk() == hd.HPC_ERR_UNSUPPORTED


def test_plan_device_argument_errors():
    lib = _lib.lib()
    ptr = ctypes.c_void_p(0x1000)
    cap = hd.hpc_decode_plan_size(4, 1, 8)
    assert lib.hpc_decode_plan_device(None, 4, 1, 8, 0, 4, ptr, cap, None) == hd.HPC_ERR_NULL
    assert lib.hpc_decode_plan_device(ptr, 4, 1, 8, 0, 4, ptr, cap - 1, None) == hd.HPC_ERR_TOO_SMALL
    assert lib.hpc_decode_plan_device(ptr, 4, 1, 0, 0, 4, ptr, cap, None) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_plan_device(ptr, 4, 1, 8, -1, 4, ptr, cap, None) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_plan_device(ptr, 4, 1, 8, hd.MAX_ENTRY_PRICE + 1, 4, ptr, cap, None) == hd.HPC_ERR_INVALID
    assert lib.hpc_decode_plan_device(ptr, 4096, 1, 8, 0, 4, ptr, 1 << 30, None) == hd.HPC_ERR_UNSUPPORTED


def test_plan_workspace_bound_covers_every_plan():
    rng = np.random.default_rng(3)
    for _ in range(40):
        B = int(rng.integers(1, 40))
        H = int(rng.choice([1, 2, 8]))
        W = int(rng.integers(1, 300))
        lens = rng.integers(0, 5000, size=B).astype(np.int32)
        plan = _cpp_plan(lens, H, W)
        bound = hd.hpc_decode_plan_workspace_bound(B, 8 * H, H, W)
        assert bound >= hd.hpc_decode_workspace_size(plan, 8 * H, H)
    assert _lib.lib().hpc_decode_plan_workspace_bound(2, 8, 1, 0) == hd.HPC_ERR_INVALID
    assert _lib.lib().hpc_decode_plan_workspace_bound(2, 12, 8, 4) == hd.HPC_ERR_INVALID


def test_plan_attn_errors_before_any_hip_call():
    """Every failure of hpc_decode_plan_attn here is found on the host before
    the plan copy or a launch is queued (no device exists in this process)."""
    lib = _lib.lib()
    ptr = 0x1000
    lens = np.asarray([37, 200], dtype=np.int32)
    H, Hq, W = 1, 8, 4
    cap = hd.hpc_decode_plan_size(2, H, W)
    host = np.zeros(cap, dtype=np.int32)
    params = hd.make_params(Hq, H, 4, 8, hd.HPC_KV_BF16, 1 / np.sqrt(128))
    need = hd.hpc_decode_workspace_size(_cpp_plan(lens, H, W), Hq, H)

    def call(lens_p=lens.ctypes.data, batch=2, w=W, ph=host.ctypes.data, c=cap, pd=ptr, sl=ptr, wsb=need,
             p=ctypes.byref(params)):
        return lib.hpc_decode_plan_attn(p, lens_p, batch, w, ph, c, pd, ptr, ptr, ptr, ptr, sl, ptr, wsb, ptr,
                                        ptr, None)
    assert call(p=None) == hd.HPC_ERR_NULL
    assert call(ph=None) == hd.HPC_ERR_NULL and call(pd=None) == hd.HPC_ERR_NULL
    assert call(pd=host.ctypes.data) == hd.HPC_ERR_INVALID           # the copy needs a separate device buffer
    assert call(lens_p=None) == hd.HPC_ERR_NULL                      # from the planner
    assert call(w=0) == hd.HPC_ERR_INVALID
    assert call(c=10) == hd.HPC_ERR_TOO_SMALL
    assert call(sl=None) == hd.HPC_ERR_NULL                          # from the attention checks
    assert call(wsb=need - 1) == hd.HPC_ERR_TOO_SMALL
    bad = np.asarray([37, 300], dtype=np.int32)                      # 5 tiles > 4 pages per sequence
    assert call(lens_p=bad.ctypes.data) == hd.HPC_ERR_INVALID
    # the planner wrote the plan of the last lengths before the check failed
    assert np.array_equal(host[:hd.hpc_decode_plan_words(host)], _cpp_plan(bad, H, W))


def test_probe_argument_errors_before_any_hip_call():
    """The measurement probes reject bad arguments on the host, before any launch."""
    lib = _lib.lib()
    ptr = 0x1000
    ms = ctypes.c_float()
    assert lib.hpc_probe_read(None, 1024, ptr, 4, None) == hd.HPC_ERR_NULL
    assert lib.hpc_probe_read(ptr, 1024, None, 4, None) == hd.HPC_ERR_NULL
    assert lib.hpc_probe_read(ptr, 1000, ptr, 4, None) == hd.HPC_ERR_INVALID     # not a multiple of 16
    assert lib.hpc_probe_read(ptr, 0, ptr, 4, None) == hd.HPC_ERR_INVALID
    assert lib.hpc_probe_read(ptr, 1024, ptr, 0, None) == hd.HPC_ERR_INVALID
    assert lib.hpc_probe_read_timed(ptr, 1024, ptr, 4, None, None) == hd.HPC_ERR_NULL
    assert lib.hpc_probe_read_timed(None, 1024, ptr, 4, None, ctypes.byref(ms)) == hd.HPC_ERR_NULL
    assert lib.hpc_probe_read_timed(ptr, 1008 + 8, ptr, 4, None, ctypes.byref(ms)) == hd.HPC_ERR_INVALID
    assert lib.hpc_probe_read_timed(ptr, 1024, ptr, -1, None, ctypes.byref(ms)) == hd.HPC_ERR_INVALID
    assert lib.hpc_probe_copy(None, ptr, 1024, None) == hd.HPC_ERR_NULL
    assert lib.hpc_probe_copy(ptr, ptr, -16, None) == hd.HPC_ERR_INVALID


def test_noalloc_step_errors_before_any_hip_call():
    """The no-allocation step refuses, on the host, shapes whose scratch
    exceeds its fixed array, the in-kernel merge and missing pointers."""
    f = hd.lib().hpc_decode_step_noalloc
    cap = hd.hpc_decode_step_noalloc_max_bytes()
    assert cap == 16 << 20
    fake = ctypes.c_void_p(0x1000)
    args = [fake] * 7
    ok = hd.make_params(16, 1, 8, 16, hd.HPC_KV_BF16, 0.088)
    assert hd.hpc_decode_step_workspace_size(2, 16, 1, 1024) > cap
    assert f(ctypes.byref(ok), 2, 1024, *args, None) == hd.HPC_ERR_TOO_SMALL
    fused = hd.make_params(16, 1, 8, 16, hd.HPC_KV_BF16, 0.088, fused_merge=True)
    assert f(ctypes.byref(fused), 2, 256, *args, None) == hd.HPC_ERR_UNSUPPORTED
    assert f(ctypes.byref(ok), 2, 256, *args[:6], None, None) == hd.HPC_ERR_NULL
    assert f(ctypes.byref(ok), 0, 256, *args, None) == hd.HPC_ERR_INVALID
    assert f(None, 2, 256, *args, None) == hd.HPC_ERR_NULL
