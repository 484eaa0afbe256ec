"""The C ABI on a host without a GPU: the library loads, exports every
symbol the header declares, and validates arguments before any HIP call."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import multiquery_decode_attention_amd as kvd
from multiquery_decode_attention_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvdecode.h")


@pytest.fixture(scope="module")
def lib():
    return kvd.library()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(kvdecode_\w+)\s*\(", text, re.M)))


def test_header_declares_the_abi():
    fns = header_functions()
    assert set(kvd.EXPORTS) == set(fns), fns


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", kvd.LIB_PATH], capture_output=True, text=True)
    for name in header_functions():
        assert re.search(rf"\bT {name}$", out.stdout, re.M), name


def test_strerror_covers_codes():
    for code in range(0, -10, -1):
        assert kvd.kvdecode_strerror(code) != "unknown status code"
    assert kvd.kvdecode_strerror(-99) == "unknown status code"


FAKE = 0x10000  # aligned address that is never dereferenced by create()


def make_desc(**kw):
    d = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, capacity=64, dtype=kvd.KVD_BF16,
             k_cache=FAKE, v_cache=FAKE * 2, lengths=FAKE * 3)
    d.update(kw)
    return kvd.kvdecode_desc_t(**d)


def create(lib, desc):
    h = ctypes.c_void_p()
    rc = lib.kvdecode_create(ctypes.byref(desc), ctypes.byref(h))
    return rc, h.value


@pytest.mark.parametrize("field,value,code", [
    ("batch", 0, kvd.KVD_EINVAL), ("batch", -3, kvd.KVD_EINVAL), ("batch", 70000, kvd.KVD_EINVAL),
    ("num_q_heads", 0, kvd.KVD_EINVAL), ("num_kv_heads", 0, kvd.KVD_EINVAL),
    ("num_q_heads", 9, kvd.KVD_EINVAL),  # not a multiple of num_kv_heads
    ("capacity", 0, kvd.KVD_EINVAL), ("capacity", (1 << 24) + 1, kvd.KVD_EINVAL),
    ("head_dim", 96, kvd.KVD_EUNSUPPORTED), ("head_dim", 512, kvd.KVD_EUNSUPPORTED),
    ("dtype", 7, kvd.KVD_EUNSUPPORTED),
    ("k_cache", 0, kvd.KVD_EINVAL), ("v_cache", 0, kvd.KVD_EINVAL), ("lengths", 0, kvd.KVD_EINVAL),
    ("k_cache", FAKE + 8, kvd.KVD_EALIGN), ("v_cache", FAKE + 2, kvd.KVD_EALIGN),
    ("lengths", FAKE + 2, kvd.KVD_EALIGN),
])
def test_create_rejects(lib, field, value, code):
    rc, h = create(lib, make_desc(**{field: value}))
    assert rc == code and not h


def test_create_null_arguments(lib):
    h = ctypes.c_void_p()
    assert lib.kvdecode_create(None, ctypes.byref(h)) == kvd.KVD_EINVAL
    assert lib.kvdecode_create(ctypes.byref(make_desc()), None) == kvd.KVD_EINVAL


def test_handle_calls_validate_before_any_device_work(lib):
    rc, h = create(lib, make_desc())
    assert rc == kvd.KVD_OK and h
    # never touched a device: status is OK without a device call
    assert lib.kvdecode_status(h, None) == kvd.KVD_OK
    # attend argument checks (no launch happens on rejection)
    assert lib.kvdecode_attend(h, None, FAKE, 1.0, None) == kvd.KVD_EINVAL
    assert lib.kvdecode_attend(h, FAKE, None, 1.0, None) == kvd.KVD_EINVAL
    assert lib.kvdecode_attend(h, FAKE + 4, FAKE, 1.0, None) == kvd.KVD_EALIGN
    assert lib.kvdecode_attend(h, FAKE, FAKE + 4, 1.0, None) == kvd.KVD_EALIGN
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert lib.kvdecode_attend(h, FAKE, FAKE, bad, None) == kvd.KVD_EINVAL
    assert lib.kvdecode_append_attend(h, None, FAKE, FAKE, FAKE, 1.0, None) == kvd.KVD_EINVAL
    assert lib.kvdecode_append_attend(h, FAKE, FAKE + 8, FAKE, FAKE, 1.0, None) == kvd.KVD_EALIGN
    assert lib.kvdecode_append_attend(h, FAKE, FAKE, None, FAKE, 1.0, None) == kvd.KVD_EINVAL
    assert lib.kvdecode_append_attend(h, FAKE, FAKE, FAKE, FAKE + 4, 1.0, None) == kvd.KVD_EALIGN
    assert lib.kvdecode_append_attend(h, FAKE, FAKE, FAKE, FAKE, float("nan"), None) == kvd.KVD_EINVAL
    for n in (0, -1, kvd.KVD_MAX_NEW_TOKENS + 1):
        assert lib.kvdecode_append_attend_multi(h, n, FAKE, FAKE, FAKE, FAKE, 1.0, None) == kvd.KVD_EINVAL
    assert lib.kvdecode_append_attend_multi(h, 2, FAKE + 8, FAKE, FAKE, FAKE, 1.0, None) == kvd.KVD_EALIGN
    assert lib.kvdecode_append_attend_multi(h, 2, FAKE, FAKE, FAKE, FAKE + 4, 1.0, None) == kvd.KVD_EALIGN
    assert lib.kvdecode_append(h, None, FAKE, None) == kvd.KVD_EINVAL
    assert lib.kvdecode_append(h, FAKE, FAKE + 8, None) == kvd.KVD_EALIGN
    # knobs
    assert lib.kvdecode_set_num_splits(h, -1) == kvd.KVD_EINVAL
    assert lib.kvdecode_set_variant(h, 9) == kvd.KVD_EUNSUPPORTED
    assert lib.kvdecode_set_variant(h, kvd.KVD_VARIANT_VALU) == kvd.KVD_OK
    assert lib.kvdecode_set_unified_max(h, 1, float("inf")) == kvd.KVD_EINVAL
    assert lib.kvdecode_set_unified_max(h, 1, float("nan")) == kvd.KVD_EINVAL
    assert lib.kvdecode_set_unified_max(h, 1, 3.5) == kvd.KVD_OK
    assert lib.kvdecode_set_unified_max(h, 0, float("nan")) == kvd.KVD_OK  # off: phi unused
    assert lib.kvdecode_reserve(h, 0) == kvd.KVD_EINVAL
    assert lib.kvdecode_reserve(h, kvd.KVD_MAX_NEW_TOKENS + 1) == kvd.KVD_EINVAL
    assert lib.kvdecode_timing_enable(h, -1, kvd.KVD_TIME_ALL) == kvd.KVD_EINVAL
    assert lib.kvdecode_timing_enable(h, 4, 8) == kvd.KVD_EINVAL
    assert lib.kvdecode_timing_enable(h, 4, kvd.KVD_TIME_ALL) == kvd.KVD_OK
    assert lib.kvdecode_timing_enable(h, 4, kvd.KVD_TIME_PARTIAL) == kvd.KVD_OK
    assert lib.kvdecode_timing_enable(h, 0, kvd.KVD_TIME_ALL) == kvd.KVD_OK
    assert lib.kvdecode_destroy(h) == kvd.KVD_OK
    # a destroyed handle is unknown to every call
    assert lib.kvdecode_destroy(h) == kvd.KVD_EINVAL
    assert lib.kvdecode_attend(h, FAKE, FAKE, 1.0, None) == kvd.KVD_EINVAL
    assert lib.kvdecode_status(h, None) == kvd.KVD_EINVAL
    assert lib.kvdecode_reserve(h, 1) == kvd.KVD_EINVAL
    assert lib.kvdecode_destroy(None) == kvd.KVD_EINVAL


def test_launch_arithmetic_is_validated(lib):
    """Shapes whose launches would not fit 32-bit grids (each grid
    dimension counts work-items in 32 bits; the kernels' row arithmetic is
    int) are refused by the step with KVD_EINVAL before any HIP call: the
    combine takes B * Hq * T_q query rows on 256-thread workgroups; the
    planner caps the split count so that the partial pass's grid fits."""
    # 65535 * 512 query rows: 2^25 of them, past 2^32 work-items
    rc, h = create(lib, make_desc(batch=65535, num_q_heads=512, num_kv_heads=1, capacity=64))
    assert rc == kvd.KVD_OK
    assert lib.kvdecode_attend(h, FAKE, FAKE, 1.0, None) == kvd.KVD_EINVAL
    assert lib.kvdecode_append_attend(h, FAKE, FAKE, FAKE, FAKE, 1.0, None) == kvd.KVD_EINVAL
    lib.kvdecode_destroy(h)
    # 65535 * 256 rows fit with one new token, not with two
    rc, h = create(lib, make_desc(batch=65535, num_q_heads=256, num_kv_heads=1, capacity=64))
    assert rc == kvd.KVD_OK
    assert lib.kvdecode_append_attend_multi(h, 2, FAKE, FAKE, FAKE, FAKE, 1.0, None) == kvd.KVD_EINVAL
    lib.kvdecode_destroy(h)
    # MHA over 65535 x 64 (sequence, head) units: a forced split count is
    # capped at the 4 splits whose grid of 256-thread workgroups fits
    rc, h = create(lib, make_desc(batch=65535, num_q_heads=64, num_kv_heads=64, capacity=65536))
    assert rc == kvd.KVD_OK
    kvd.kvdecode_set_num_splits(h, 10**6)
    units = -(-65535 * 64 // 8) * 8
    assert kvd.kvdecode_get_plan(h)["num_splits"] == (2**32 - 1) // (256 * units) == 4
    lib.kvdecode_destroy(h)


def test_noalloc_step_refuses_what_its_buffer_cannot_hold(lib):
    """The allocation-free step checks its arguments like the allocating
    one, and refuses (KVD_ESCRATCH) a step whose workspace exceeds the
    static buffer, all before any HIP call."""
    rc, h = create(lib, make_desc())
    assert rc == kvd.KVD_OK
    f = lib.kvdecode_append_attend_noalloc
    assert f(h, None, FAKE, FAKE, FAKE, 1.0, None) == kvd.KVD_EINVAL
    assert f(h, FAKE, FAKE + 8, FAKE, FAKE, 1.0, None) == kvd.KVD_EALIGN
    assert f(h, FAKE, FAKE, None, FAKE, 1.0, None) == kvd.KVD_EINVAL
    assert f(h, FAKE, FAKE, FAKE, FAKE + 4, 1.0, None) == kvd.KVD_EALIGN
    assert f(h, FAKE, FAKE, FAKE, FAKE, float("nan"), None) == kvd.KVD_EINVAL
    lib.kvdecode_destroy(h)
    assert f(h, FAKE, FAKE, FAKE, FAKE, 1.0, None) == kvd.KVD_EINVAL  # destroyed handle
    # 4096 x 48 heads x 256 columns of bf16 partials at one split already
    # take 96 MiB, past the 32 MiB buffer
    rc, h = create(lib, make_desc(batch=4096, num_q_heads=48, num_kv_heads=1, head_dim=256, capacity=2048))
    assert rc == kvd.KVD_OK
    kvd.kvdecode_set_num_splits(h, 1)
    assert f(h, FAKE, FAKE, FAKE, FAKE, 1.0, None) == kvd.KVD_ESCRATCH
    lib.kvdecode_destroy(h)


def test_mfma_variant_needs_bf16(lib):
    rc, h = create(lib, make_desc(dtype=kvd.KVD_F32))
    assert rc == kvd.KVD_OK
    assert lib.kvdecode_set_variant(h, kvd.KVD_VARIANT_MFMA) == kvd.KVD_EUNSUPPORTED
    assert kvd.kvdecode_get_plan(h)["variant"] == "valu"
    lib.kvdecode_destroy(h)


def plan_of(lib, **kw):
    rc, h = create(lib, make_desc(**kw))
    assert rc == kvd.KVD_OK
    try:
        return kvd.kvdecode_get_plan(h), h
    finally:
        pass


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_plans_cover_the_cache(lib, name):
    w = inputs.WORKLOADS[name]
    dt = kvd.KVD_F32 if w.dtype == "f32" else kvd.KVD_BF16
    for forced in (0, 1, 2, 7, 10**6):
        rc, h = create(lib, make_desc(batch=w.B, num_q_heads=w.Hq, num_kv_heads=w.Hkv, head_dim=w.D,
                                      capacity=w.T_cap, dtype=dt))
        assert rc == kvd.KVD_OK
        kvd.kvdecode_set_num_splits(h, forced)
        p = kvd.kvdecode_get_plan(h)
        tile = 64 if p["variant"] == "valu" else 32
        S, C = p["num_splits"], p["split_tokens"]
        assert C % tile == 0 and S >= 1
        n_tiles = -(-w.T_cap // tile)
        assert S * C >= w.T_cap and S <= n_tiles
        assert C == -(-n_tiles // S) * tile  # round-robin tiles: the busiest split
        if forced:
            assert S <= forced or S == 1
        lib.kvdecode_destroy(h)


def make_paged_desc(**kw):
    d = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=64, num_pages=10,
             max_pages=4, dtype=kvd.KVD_BF16, k_pages=FAKE, v_pages=FAKE * 2, block_table=FAKE * 3,
             lengths=FAKE * 4)
    d.update(kw)
    return kvd.kvdecode_paged_desc_t(**d)


def create_paged(lib, desc):
    h = ctypes.c_void_p()
    rc = lib.kvdecode_create_paged(ctypes.byref(desc), ctypes.byref(h))
    return rc, h.value


@pytest.mark.parametrize("field,value,code", [
    ("page_size", 16, kvd.KVD_EINVAL), ("page_size", 48, kvd.KVD_EINVAL),
    ("page_size", 1 << 17, kvd.KVD_EINVAL), ("page_size", 0, kvd.KVD_EINVAL),
    ("num_pages", 0, kvd.KVD_EINVAL), ("max_pages", 0, kvd.KVD_EINVAL),
    ("max_pages", (1 << 18) + 1, kvd.KVD_EINVAL),       # capacity past 2^24
    ("num_pages", (1 << 24) + 1, kvd.KVD_EINVAL),       # pool rows past 2^31
    ("block_table", 0, kvd.KVD_EINVAL), ("block_table", FAKE + 2, kvd.KVD_EALIGN),
    ("k_pages", 0, kvd.KVD_EINVAL), ("v_pages", FAKE + 8, kvd.KVD_EALIGN),
    ("head_dim", 96, kvd.KVD_EUNSUPPORTED), ("num_q_heads", 9, kvd.KVD_EINVAL),
])
def test_create_paged_rejects(lib, field, value, code):
    rc, h = create_paged(lib, make_paged_desc(**{field: value}))
    assert rc == code and not h


def test_paged_handle(lib):
    rc, h = create_paged(lib, make_paged_desc())
    assert rc == kvd.KVD_OK and h
    # capacity is max_pages * page_size; the register-direct MFMA kernel has no paged mode
    assert lib.kvdecode_set_variant(h, kvd.KVD_VARIANT_MFMA) == kvd.KVD_EUNSUPPORTED
    assert lib.kvdecode_set_variant(h, kvd.KVD_VARIANT_VALU) == kvd.KVD_OK
    p = kvd.kvdecode_get_plan(h)
    assert p["variant"] == "valu" and p["num_splits"] * p["split_tokens"] >= 4 * 64
    assert lib.kvdecode_set_variant(h, kvd.KVD_VARIANT_AUTO) == kvd.KVD_OK
    assert kvd.kvdecode_get_plan(h)["variant"] == "lds"
    assert lib.kvdecode_attend(h, FAKE + 4, FAKE, 1.0, None) == kvd.KVD_EALIGN
    assert lib.kvdecode_status(h, None) == kvd.KVD_OK
    assert lib.kvdecode_destroy(h) == kvd.KVD_OK
    assert lib.kvdecode_create_paged(None, ctypes.byref(ctypes.c_void_p())) == kvd.KVD_EINVAL


def test_binding_fails_loudly_without_library(tmp_path):
    code = (
        "import multiquery_decode_attention_amd as k\n"
        f"k.LIB_PATH = {str(tmp_path / 'missing.so')!r}\n"
        "k._lib = None\n"
        "try:\n"
        "    k.library()\n"
        "except k.KvdLibraryMissing:\n"
        "    print('missing-raised')\n"
    )
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert "missing-raised" in r.stdout, r.stderr


def make_fp8_desc(**kw):
    cache = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, capacity=64,
                 dtype=kvd.KVD_FP8_E4M3, k_cache=FAKE, v_cache=FAKE * 2, lengths=FAKE * 3)
    exps = dict(k_exp=FAKE * 4, v_exp=FAKE * 5)
    for k, v in kw.items():
        (exps if k in exps else cache)[k] = v
    return kvd.kvdecode_fp8_desc_t(kvd.kvdecode_desc_t(**cache), exps["k_exp"], exps["v_exp"])


@pytest.mark.parametrize("field,value,code", [
    ("capacity", 48, kvd.KVD_EINVAL), ("capacity", 0, kvd.KVD_EINVAL),
    ("k_exp", 0, kvd.KVD_EINVAL), ("v_exp", FAKE + 4, kvd.KVD_EALIGN),
    ("dtype", kvd.KVD_BF16, kvd.KVD_EUNSUPPORTED), ("head_dim", 96, kvd.KVD_EUNSUPPORTED),
])
def test_create_fp8_rejects(lib, field, value, code):
    h = ctypes.c_void_p()
    rc = lib.kvdecode_create_fp8(ctypes.byref(make_fp8_desc(**{field: value})), ctypes.byref(h))
    assert rc == code and not h.value


def test_fp8_handle(lib):
    h = ctypes.c_void_p()
    assert lib.kvdecode_create_fp8(ctypes.byref(make_fp8_desc()), ctypes.byref(h)) == kvd.KVD_OK
    assert kvd.kvdecode_get_plan(h.value)["variant"] == "wave"  # d = 128
    for v in (kvd.KVD_VARIANT_VALU, kvd.KVD_VARIANT_MFMA):
        assert lib.kvdecode_set_variant(h.value, v) == kvd.KVD_EUNSUPPORTED
    assert lib.kvdecode_set_variant(h.value, kvd.KVD_VARIANT_LDS) == kvd.KVD_OK
    assert kvd.kvdecode_get_plan(h.value)["variant"] == "lds"
    assert lib.kvdecode_set_variant(h.value, kvd.KVD_VARIANT_WAVE) == kvd.KVD_OK
    assert kvd.kvdecode_get_plan(h.value)["variant"] == "wave"
    # the exchange kernel walks 64-token tiles: its splits hold multiples of 64
    assert lib.kvdecode_set_variant(h.value, kvd.KVD_VARIANT_XCHG) == kvd.KVD_OK
    p = kvd.kvdecode_get_plan(h.value)
    assert p["variant"] == "xchg" and p["split_tokens"] % 64 == 0
    assert lib.kvdecode_destroy(h.value) == kvd.KVD_OK
    # d = 64: the wave and exchange kernels need 16-byte code chunks of the value rows
    assert lib.kvdecode_create_fp8(ctypes.byref(make_fp8_desc(head_dim=64)), ctypes.byref(h)) == kvd.KVD_OK
    assert kvd.kvdecode_get_plan(h.value)["variant"] == "lds"
    assert lib.kvdecode_set_variant(h.value, kvd.KVD_VARIANT_WAVE) == kvd.KVD_EUNSUPPORTED
    assert lib.kvdecode_set_variant(h.value, kvd.KVD_VARIANT_XCHG) == kvd.KVD_EUNSUPPORTED
    assert lib.kvdecode_destroy(h.value) == kvd.KVD_OK
    # groups above 16 query rows at d = 256 take the exchange kernel
    assert lib.kvdecode_create_fp8(ctypes.byref(make_fp8_desc(head_dim=256, num_q_heads=48, num_kv_heads=1)),
                                   ctypes.byref(h)) == kvd.KVD_OK
    assert kvd.kvdecode_get_plan(h.value)["variant"] == "xchg"
    assert lib.kvdecode_destroy(h.value) == kvd.KVD_OK
    # bf16 and fp32 handles: neither fp8 kernel
    for desc in (make_desc(), make_desc(head_dim=64), make_desc(dtype=kvd.KVD_F32)):
        rc, hb = create(lib, desc)
        assert rc == kvd.KVD_OK
        for v in (kvd.KVD_VARIANT_WAVE, kvd.KVD_VARIANT_XCHG):
            assert lib.kvdecode_set_variant(hb, v) == kvd.KVD_EUNSUPPORTED
        assert lib.kvdecode_destroy(hb) == kvd.KVD_OK
    # the fp8 cache type is only reachable through kvdecode_create_fp8
    rc, h2 = create(lib, make_desc(dtype=kvd.KVD_FP8_E4M3))
    assert rc == kvd.KVD_EUNSUPPORTED and not h2
    rc, h3 = create_paged(lib, make_paged_desc(dtype=kvd.KVD_FP8_E4M3))
    assert rc == kvd.KVD_EUNSUPPORTED and not h3


def make_fp8_paged_desc(**kw):
    exps = dict(k_exp=FAKE * 5, v_exp=FAKE * 6)
    pages = dict(dtype=kvd.KVD_FP8_E4M3)
    for k, v in kw.items():
        (exps if k in exps else pages)[k] = v
    return kvd.kvdecode_fp8_paged_desc_t(make_paged_desc(**pages), exps["k_exp"], exps["v_exp"])


@pytest.mark.parametrize("field,value,code", [
    ("page_size", 16, kvd.KVD_EINVAL), ("num_pages", 0, kvd.KVD_EINVAL),
    ("block_table", FAKE + 2, kvd.KVD_EALIGN), ("k_exp", 0, kvd.KVD_EINVAL),
    ("v_exp", FAKE + 4, kvd.KVD_EALIGN), ("dtype", kvd.KVD_BF16, kvd.KVD_EUNSUPPORTED),
    ("head_dim", 96, kvd.KVD_EUNSUPPORTED),
])
def test_create_fp8_paged_rejects(lib, field, value, code):
    h = ctypes.c_void_p()
    rc = lib.kvdecode_create_fp8_paged(ctypes.byref(make_fp8_paged_desc(**{field: value})), ctypes.byref(h))
    assert rc == code and not h.value


def test_fp8_paged_handle(lib):
    h = ctypes.c_void_p()
    assert lib.kvdecode_create_fp8_paged(ctypes.byref(make_fp8_paged_desc()), ctypes.byref(h)) == kvd.KVD_OK
    p = kvd.kvdecode_get_plan(h.value)
    assert p["variant"] == "wave" and p["num_splits"] * p["split_tokens"] >= 4 * 64
    assert lib.kvdecode_set_variant(h.value, kvd.KVD_VARIANT_LDS) == kvd.KVD_OK
    for v in (kvd.KVD_VARIANT_VALU, kvd.KVD_VARIANT_MFMA):
        assert lib.kvdecode_set_variant(h.value, v) == kvd.KVD_EUNSUPPORTED
    assert lib.kvdecode_destroy(h.value) == kvd.KVD_OK
    # the fp8 dtype needs the fp8 create call, and that call the fp8 dtype
    rc, h2 = create_paged(lib, make_paged_desc(dtype=kvd.KVD_FP8_E4M3))
    assert rc == kvd.KVD_EUNSUPPORTED and not h2
    assert lib.kvdecode_create_fp8_paged(None, ctypes.byref(ctypes.c_void_p())) == kvd.KVD_EINVAL


def test_plan_of_several_new_tokens(lib):
    """kvdecode_get_plan_multi: one token reports kvdecode_get_plan's plan;
    a step's query rows grow with n_tokens, and the plan may change with
    them (the PaLM-like batch: 4 splits for one token, 2 for four); counts
    outside 1..KVD_MAX_NEW_TOKENS and the one-token MFMA kernel are refused."""
    rc, h = create(lib, make_desc(batch=64, num_q_heads=48, num_kv_heads=1, head_dim=256, capacity=2048))
    assert rc == kvd.KVD_OK
    try:
        assert kvd.kvdecode_get_plan_multi(h, 1) == kvd.kvdecode_get_plan(h)
        assert kvd.kvdecode_get_plan(h)["num_splits"] == 4
        assert kvd.kvdecode_get_plan_multi(h, 4)["num_splits"] == 2
        v, s, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        for n in (0, -1, kvd.KVD_MAX_NEW_TOKENS + 1):
            assert lib.kvdecode_get_plan_multi(h, n, ctypes.byref(v), ctypes.byref(s), ctypes.byref(c)) == kvd.KVD_EINVAL
        assert lib.kvdecode_get_plan_multi(h, 2, None, None, None) == kvd.KVD_OK
        assert lib.kvdecode_set_variant(h, kvd.KVD_VARIANT_MFMA) == kvd.KVD_OK
        assert lib.kvdecode_get_plan_multi(h, 1, None, None, None) == kvd.KVD_OK
        assert lib.kvdecode_get_plan_multi(h, 2, None, None, None) == kvd.KVD_EUNSUPPORTED
    finally:
        lib.kvdecode_destroy(h)
    assert lib.kvdecode_get_plan_multi(None, 1, None, None, None) == kvd.KVD_EINVAL
