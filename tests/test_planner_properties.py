"""Property tests of the host side of the C ABI (CPU, no device calls):
for any cache description the library accepts, the split plan covers the
cache with whole tiles, holds at most one split per tile, never exceeds a
forced split count, is the same when asked again, and uses the kernel the
header documents for the cache type; descriptions outside the documented
limits are refused without a handle."""
import ctypes

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import multiquery_decode_attention_amd as kvd

FAKE = 0x10000  # aligned address that create() never dereferences
SETTINGS = settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
VARIANT_NAMES = {1: "valu", 2: "mfma", 3: "lds", 4: "wave", 5: "xchg"}


@pytest.fixture(scope="module")
def lib():
    return kvd.library()


def desc(B, Hq, Hkv, D, T_cap, dtype):
    return kvd.kvdecode_desc_t(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, capacity=T_cap,
                               dtype=dtype, k_cache=FAKE, v_cache=FAKE * 2, lengths=FAKE * 3)


def create(lib, B, Hq, Hkv, D, T_cap, dtype):
    h = ctypes.c_void_p()
    if dtype == kvd.KVD_FP8_E4M3:
        d = kvd.kvdecode_fp8_desc_t(cache=desc(B, Hq, Hkv, D, T_cap, dtype), k_exp=FAKE * 4, v_exp=FAKE * 5)
        rc = lib.kvdecode_create_fp8(ctypes.byref(d), ctypes.byref(h))
    else:
        d = desc(B, Hq, Hkv, D, T_cap, dtype)
        rc = lib.kvdecode_create(ctypes.byref(d), ctypes.byref(h))
    return rc, h.value


def plan(lib, h, T_q=1):
    v, s, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    assert lib.kvdecode_get_plan_multi(h, T_q, ctypes.byref(v), ctypes.byref(s), ctypes.byref(c)) == kvd.KVD_OK
    if T_q == 1:
        v1, s1, c1 = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        assert lib.kvdecode_get_plan(h, ctypes.byref(v1), ctypes.byref(s1), ctypes.byref(c1)) == kvd.KVD_OK
        assert (v1.value, s1.value, c1.value) == (v.value, s.value, c.value)
    return VARIANT_NAMES[v.value], s.value, c.value


@st.composite
def caches(draw):
    dtype = draw(st.sampled_from([kvd.KVD_F32, kvd.KVD_BF16, kvd.KVD_FP8_E4M3]))
    D = draw(st.sampled_from([64, 128, 256]))
    Hkv = draw(st.integers(1, 64))
    M = draw(st.integers(1, 96))
    B = draw(st.integers(1, 2048))
    # fp8 capacities are whole 32-token blocks (the exponent loads read 16 rows at once)
    T_cap = draw(st.integers(1, 1 << 16)) if dtype != kvd.KVD_FP8_E4M3 else 32 * draw(st.integers(1, 2048))
    return B, Hkv * M, Hkv, D, T_cap, dtype


@SETTINGS
@given(caches(), st.integers(0, 5000), st.integers(1, kvd.KVD_MAX_NEW_TOKENS))
def test_plan_properties(lib, cache, forced, T_q):
    """Plans of steps with T_q new tokens (the query rows per KV head grow
    with T_q)."""
    B, Hq, Hkv, D, T_cap, dtype = cache
    rc, h = create(lib, B, Hq, Hkv, D, T_cap, dtype)
    assert rc == kvd.KVD_OK and h
    try:
        assert lib.kvdecode_set_num_splits(h, forced) == kvd.KVD_OK
        variant, S, C = plan(lib, h, T_q)
        assert plan(lib, h, T_q) == (variant, S, C)  # cached, stable
        # the automatic kernel choice the header documents
        rows = Hq // Hkv * T_q
        if dtype == kvd.KVD_F32:
            assert variant == "valu"
        elif dtype == kvd.KVD_BF16:
            assert variant == "lds"
        elif D < 128:
            assert variant == "lds"
        else:
            assert variant == ("wave" if rows <= (16 if D == 256 else 48) else "xchg")
        tile = {"valu": 64, "xchg": 64}.get(variant, 32)
        n_tiles = -(-T_cap // tile)
        # whole tiles dealt round-robin: S splits, at most one per tile, the
        # busiest holding ceil(n_tiles / S) of them
        assert 1 <= S <= n_tiles
        assert C == -(-n_tiles // S) * tile and S * C >= T_cap
        if forced:
            assert S <= forced
    finally:
        assert lib.kvdecode_destroy(h) == kvd.KVD_OK


@SETTINGS
@given(st.integers(-5, 70000), st.integers(-3, 300), st.integers(-3, 300), st.sampled_from([0, 32, 64, 96, 128, 256, 512]),
       st.integers(-5, (1 << 24) + 5), st.sampled_from([-1, 0, 1, 2, 3]))
def test_create_accepts_exactly_the_documented_descriptions(lib, B, Hq, Hkv, D, T_cap, dtype):
    """kvdecode_create on the contiguous layout: accepted exactly when every
    field lies in the documented range (1 <= B <= 65535, heads positive
    with Hq a multiple of Hkv, d in {64, 128, 256}, 1 <= capacity <= 2^24,
    a known dtype; fp8 has its own create call), else a negative code and
    no handle."""
    valid_shape = (1 <= B <= 65535 and Hq >= 1 and Hkv >= 1 and Hq % Hkv == 0 and 1 <= T_cap <= (1 << 24))
    d = desc(B, Hq, Hkv, D, T_cap, dtype)
    h = ctypes.c_void_p()
    rc = lib.kvdecode_create(ctypes.byref(d), ctypes.byref(h))
    if rc == kvd.KVD_OK:
        assert h.value
        assert valid_shape and D in (64, 128, 256) and dtype in (kvd.KVD_F32, kvd.KVD_BF16)
        assert lib.kvdecode_destroy(h.value) == kvd.KVD_OK
    else:
        assert rc < 0 and not h.value
        assert not (valid_shape and D in (64, 128, 256) and dtype in (kvd.KVD_F32, kvd.KVD_BF16))
