"""Pins of the several-new-tokens (speculative-verify) oracle.

One new token reduces to the single-token step; a sequence grown in steps
of T_q tokens gives every query the same output as a full causal softmax
over the whole sequence computed from scratch (the definition of causal
attention, written independently here); a sequence that cannot take T_q
more tokens is left unchanged and its queries see the cache as it stands.
"""
import numpy as np
import pytest

import oracle


def _rand(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


def test_one_new_token_is_the_single_token_step():
    rng = np.random.default_rng(1)
    B, Hq, Hkv, T, D = 3, 8, 2, 20, 16
    k, v = _rand(rng, B, Hkv, T, D), _rand(rng, B, Hkv, T, D)
    kn, vn, q = _rand(rng, B, Hkv, 1, D), _rand(rng, B, Hkv, 1, D), _rand(rng, B, Hq, 1, D)
    L0 = np.array([0, 7, 19])
    k2, v2, L2, a = oracle.append_multi(k, v, L0, kn, vn)
    k1, v1, L1, _ = oracle.append(k, v, L0, kn[:, :, 0], vn[:, :, 0])
    assert np.array_equal(k2, k1) and np.array_equal(v2, v1) and np.array_equal(L2, L1)
    got = oracle.decode_attention_multi(q, k2, v2, L2, a, 0.25, oracle.F32)[:, :, 0]
    want = oracle.decode_attention(q[:, :, 0], k1, v1, L1, 0.25, oracle.F32)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("T_q", [2, 3, 5])
def test_steps_of_several_tokens_match_full_causal_attention(T_q):
    rng = np.random.default_rng(T_q)
    Hq, Hkv, D, steps = 4, 2, 8, 4
    T = T_q * steps
    K, V, Q = _rand(rng, T, Hkv, D), _rand(rng, T, Hkv, D), _rand(rng, T, Hq, D)
    scale = 0.4
    # full causal attention from scratch, fp64: token t attends to 0..t
    full = np.zeros((T, Hq, D))
    for t in range(T):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            s = scale * (K[:t + 1, g].astype(np.float64) @ Q[t, h].astype(np.float64))
            p = np.exp(s - s.max())
            full[t, h] = (p / p.sum()) @ V[:t + 1, g].astype(np.float64)
    k = np.full((1, Hkv, T, D), np.nan, np.float32)
    v = np.full((1, Hkv, T, D), np.nan, np.float32)
    L = np.array([0])
    for st in range(steps):
        sl = slice(st * T_q, (st + 1) * T_q)
        kn = K[sl].transpose(1, 0, 2)[None]
        vn = V[sl].transpose(1, 0, 2)[None]
        q = Q[sl].transpose(1, 0, 2)[None]
        k, v, L, a = oracle.append_multi(k, v, L, kn, vn)
        got = oracle.decode_attention_multi(q, k, v, L, a, scale, oracle.F32)[0]  # [Hq, T_q, D]
        assert np.allclose(got.transpose(1, 0, 2), full[sl], rtol=1e-5, atol=1e-6)
    assert L.tolist() == [T]


def test_sequence_without_room_is_left_unchanged():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, T, D, T_q = 2, 4, 1, 10, 8, 3
    k, v = _rand(rng, B, Hkv, T, D), _rand(rng, B, Hkv, T, D)
    kn, vn, q = _rand(rng, B, Hkv, T_q, D), _rand(rng, B, Hkv, T_q, D), _rand(rng, B, Hq, T_q, D)
    k2, v2, L2, a = oracle.append_multi(k, v, np.array([8, 7]), kn, vn)
    assert L2.tolist() == [8, 10] and a.tolist() == [0, 3]
    assert np.array_equal(k2[0], k[0]) and np.array_equal(k2[1, :, 7:], kn[1])
    out = oracle.decode_attention_multi(q, k2, v2, L2, a, 0.5, oracle.F32)
    # every query of the full sequence sees its 8 cached tokens
    for i in range(T_q):
        want = oracle.decode_attention(np.ascontiguousarray(q[:, :, i]), k2, v2, np.array([8, 8]), 0.5, oracle.F32)
        assert np.array_equal(out[0, :, i], want[0])


MULTI_MUTANTS = {
    "query_sees_next_token": ("Li = (L - a + np.minimum(i + 1, a))", "Li = (L - a + np.minimum(i + 2, a))"),
    "query_blind_to_itself": ("Li = (L - a + np.minimum(i + 1, a))", "Li = (L - a + np.minimum(i, a))"),
    "rows_reversed": ("k2[b, :, n[b] + i, :] = k_new[b, :, i]", "k2[b, :, n[b] + i, :] = k_new[b, :, T_q - 1 - i]"),
    "partial_append": ("if n[b] < 0 or n[b] + T_q > T_cap:", "if n[b] < 0 or n[b] >= T_cap:"),
}


@pytest.mark.parametrize("name", sorted(MULTI_MUTANTS))
def test_multi_mutant_is_caught(name, monkeypatch):
    import inspect
    import types
    old, new = MULTI_MUTANTS[name]
    src = inspect.getsource(oracle)
    assert src.count(old) == 1, old
    m = types.ModuleType("oracle_multi_mutant")
    m.__file__ = oracle.__file__
    exec(compile(src.replace(old, new), "oracle_multi_mutant", "exec"), m.__dict__)
    failed = []
    for pin, args in ((test_one_new_token_is_the_single_token_step, ()),
                      (test_steps_of_several_tokens_match_full_causal_attention, (3,)),
                      (test_sequence_without_room_is_left_unchanged, ())):
        with monkeypatch.context() as mp:
            mp.setattr(oracle, "append_multi", m.append_multi)
            mp.setattr(oracle, "decode_attention_multi", m.decode_attention_multi)
            try:
                pin(*args)
            except (AssertionError, IndexError, ValueError):
                failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


# --- fp8 cache ------------------------------------------------------------------

def _fp8_cache(rng, B, Hkv, T, D):
    codes = [rng.integers(0, 0x7E, (B, Hkv, T, D)).astype(np.uint8) for _ in range(2)]
    exps = [rng.integers(-9, -4, (B, Hkv, T)).astype(np.int8) for _ in range(2)]
    return codes[0], exps[0], codes[1], exps[1]


def test_fp8_one_new_token_is_the_single_token_fp8_step():
    rng = np.random.default_rng(21)
    B, Hq, Hkv, T, D = 3, 4, 2, 12, 8
    cache = _fp8_cache(rng, B, Hkv, T, D)
    kn, vn = rng.standard_normal((B, Hkv, D)), rng.standard_normal((B, Hkv, D)) * 30
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    L = np.array([0, 5, 12])
    one = oracle.append_fp8(*cache, L, kn, vn)
    multi = oracle.append_fp8_multi(*cache, L, kn[:, :, None], vn[:, :, None])
    for a, b in zip(one[:5], multi[:5]):
        assert np.array_equal(a, b)
    assert multi[5].tolist() == [1, 1, 0]
    want = oracle.decode_attention_fp8(q, *one[:5], 0.4)
    got = oracle.decode_attention_fp8_multi(q[:, :, None], *multi[:5], multi[5], 0.4)[:, :, 0]
    assert np.array_equal(got, want)


def test_fp8_several_tokens_are_successive_single_appends():
    """T_q rows appended at once equal T_q single-token fp8 appends, and
    query i sees the cache up to its own token only."""
    rng = np.random.default_rng(22)
    B, Hq, Hkv, T, D, T_q = 3, 4, 1, 16, 8, 4
    cache = _fp8_cache(rng, B, Hkv, T, D)
    kn, vn = rng.standard_normal((B, Hkv, T_q, D)), rng.standard_normal((B, Hkv, T_q, D))
    q = rng.standard_normal((B, Hq, T_q, D)).astype(np.float32)
    L = np.array([3, 12, 14])  # the last has no room for 4
    multi = oracle.append_fp8_multi(*cache, L, kn, vn)
    assert multi[5].tolist() == [4, 4, 0] and multi[4].tolist() == [7, 16, 14]
    state, n = [x[:2] for x in cache], L[:2]  # the two sequences with room, one token at a time
    for i in range(T_q):
        *state, n, _ = oracle.append_fp8(*state, n, kn[:2, :, i], vn[:2, :, i])
    assert n.tolist() == [7, 16]
    for a, b in zip(state, multi[:4]):
        assert np.array_equal(a, b[:2])
    for x, c in zip(multi[:4], cache):
        assert np.array_equal(x[2], c[2])  # the full sequence is unchanged
    out = oracle.decode_attention_fp8_multi(q, *multi[:5], multi[5], 0.5)
    for i in range(T_q):
        Li = np.array([3 + i + 1, 12 + i + 1, 14])
        want = oracle.decode_attention_fp8(np.ascontiguousarray(q[:, :, i]), *multi[:4], Li, 0.5)
        assert np.array_equal(out[:, :, i], want)


FP8_MULTI_MUTANTS = {
    "fp8_rows_reversed": ("kc[b, :, n[b] + i, :], ke[b, :, n[b] + i] = qk[b, :, i], ek[b, :, i]",
                          "kc[b, :, n[b] + i, :], ke[b, :, n[b] + i] = qk[b, :, T_q - 1 - i], ek[b, :, T_q - 1 - i]"),
    "fp8_partial_append": ("if n[b] < 0 or T_cap - n[b] < T_q:", "if n[b] < 0 or T_cap - n[b] < 1:"),
    "fp8_exponent_of_first_row": ("vc[b, :, n[b] + i, :], ve[b, :, n[b] + i] = qv[b, :, i], ev[b, :, i]",
                                  "vc[b, :, n[b] + i, :], ve[b, :, n[b] + i] = qv[b, :, i], ev[b, :, 0]"),
}


@pytest.mark.parametrize("name", sorted(FP8_MULTI_MUTANTS))
def test_fp8_multi_mutant_is_caught(name, monkeypatch):
    import inspect
    import types
    old, new = FP8_MULTI_MUTANTS[name]
    src = inspect.getsource(oracle)
    assert src.count(old) == 1, old
    m = types.ModuleType("oracle_fp8_multi_mutant")
    m.__file__ = oracle.__file__
    exec(compile(src.replace(old, new), "oracle_fp8_multi_mutant", "exec"), m.__dict__)
    failed = []
    for pin in (test_fp8_one_new_token_is_the_single_token_fp8_step, test_fp8_several_tokens_are_successive_single_appends):
        with monkeypatch.context() as mp:
            mp.setattr(oracle, "append_fp8_multi", m.append_fp8_multi)
            mp.setattr(oracle, "decode_attention_fp8_multi", m.decode_attention_fp8_multi)
            try:
                pin()
            except (AssertionError, IndexError, ValueError):
                failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
