"""Pins of the CPU oracle against facts that do not come from the oracle.

Each pin is a function ``pin(lib)`` that raises AssertionError when the
oracle library ``lib`` (the real one, or a build with a planted mistake)
disagrees with:

* exact values worked by hand (tests/golden/hand_worked_attention.json);
* closed forms: one cached token returns its value; identical keys or a
  zero query return the mean of the values; a huge scale returns the value
  of the best-scoring key;
* invariants of the definition: multiquery == multi-head with replicated
  K/V, grouped-query == independent multiquery problems per KV head,
  permuting the valid tokens, adding one vector to every key, rescaling the
  query against the scale, and never reading slots past the valid length;
* a 50-digit brute-force evaluation (mpmath, no max subtraction);
* naive recomputation of full causal attention over the whole prefix at
  every step ("All About Transformer Inference", section "Transformer
  inference basics": the KV cache avoids reprocessing earlier tokens, so
  cached decoding must reproduce recomputation).
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "hand_worked_attention.json")


def _to_bits_bf16(x32: np.ndarray) -> np.ndarray:
    """Exact bf16 encoding of fp32 values that bf16 represents exactly."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def _run(lib, q, k, v, lengths, scale, dtype=oracle.F32):
    if dtype == oracle.BF16:
        q, k, v = _to_bits_bf16(q), _to_bits_bf16(k), _to_bits_bf16(v)
    return oracle.decode_attention(q, k, v, lengths, scale, dtype, lib=lib, threads=2)


def _rand(rng, shape, grid=None):
    """N(0,1) fp32 draws; with ``grid`` rounded to multiples of 1/grid
    (exact in bf16 for small magnitudes)."""
    x = rng.standard_normal(shape)
    if grid:
        x = np.round(x * grid) / grid
    return x.astype(np.float32)


def golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def pin_golden(lib):
    for case in golden_cases():
        for dtype in (oracle.F32, oracle.BF16):
            q = np.array(case["q"], dtype=np.float32)
            k = np.array(case["k"], dtype=np.float32)
            v = np.array(case["v"], dtype=np.float32)
            L = np.array(case["lengths"], dtype=np.int32)
            if case.get("poison_tail"):
                for b, n in enumerate(L):
                    k[b, :, n:, :] = np.nan
                    v[b, :, n:, :] = np.nan
            scale = eval(case["scale_expr"], {"log": math.log})  # noqa: S307 (fixture-owned)
            if dtype == oracle.BF16 and case.get("poison_tail"):
                # NaN has a bf16 encoding; keep the quiet-NaN pattern
                pass
            got = _run(lib, q, k, v, L, scale, dtype)
            want = np.array([[[float(Fraction(x)) for x in row] for row in hb] for hb in case["out"]])
            assert np.allclose(got, want, rtol=1e-12, atol=1e-12), (case["id"], got, want)


def pin_single_token(lib):
    rng = np.random.default_rng(11)
    B, Hq, Hkv, D, T = 3, 6, 2, 16, 5
    q, k, v = _rand(rng, (B, Hq, D)), _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
    L = np.ones(B, np.int32)
    got = _run(lib, q, k, v, L, 0.37)
    M = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            assert np.array_equal(got[b, h], v[b, h // M, 0].astype(np.float64)), (b, h)


def pin_identical_keys_mean(lib):
    rng = np.random.default_rng(12)
    B, Hq, Hkv, D, T = 2, 4, 1, 8, 7
    q, v = _rand(rng, (B, Hq, D)), _rand(rng, (B, Hkv, T, D))
    k = np.repeat(_rand(rng, (B, Hkv, 1, D)), T, axis=2)
    L = np.array([7, 4], np.int32)
    got = _run(lib, q, k, v, L, 1.3)
    for b in range(B):
        mean = v[b, 0, :L[b]].astype(np.float64).mean(axis=0)
        for h in range(Hq):
            assert np.allclose(got[b, h], mean, rtol=1e-12, atol=1e-13), (b, h)


def pin_zero_query_mean(lib):
    rng = np.random.default_rng(13)
    B, Hq, Hkv, D, T = 2, 4, 2, 8, 6
    q = np.zeros((B, Hq, D), np.float32)
    k, v = _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
    L = np.array([6, 3], np.int32)
    got = _run(lib, q, k, v, L, 0.5)
    for b in range(B):
        for h in range(Hq):
            mean = v[b, h // 2, :L[b]].astype(np.float64).mean(axis=0)
            assert np.allclose(got[b, h], mean, rtol=1e-12, atol=1e-13), (b, h)


def pin_argmax_limit(lib):
    # scores on a 1/4 grid, scaled by 1e4: every non-maximal weight underflows.
    rng = np.random.default_rng(14)
    B, Hq, Hkv, D, T = 1, 3, 1, 4, 6
    k = _rand(rng, (B, Hkv, T, D), grid=4)
    v = _rand(rng, (B, Hkv, T, D))
    q = _rand(rng, (B, Hq, D), grid=4)
    L = np.array([T], np.int32)
    s = (q[0].astype(np.float64) @ k[0, 0].astype(np.float64).T)  # [Hq, T]
    got = _run(lib, q, k, v, L, 1e4)
    for h in range(Hq):
        best = np.sort(s[h])
        if best[-1] - best[-2] < 0.05:
            continue  # tie: the limit is an average, not a single row
        assert np.array_equal(got[0, h], v[0, 0, int(np.argmax(s[h]))].astype(np.float64)), h
    # the opposite limit (scale -> 0) is the mean
    got0 = _run(lib, q, k, v, L, 1e-30)
    assert np.allclose(got0[0], v[0, 0].astype(np.float64).mean(0), rtol=1e-12, atol=1e-13)


def pin_mqa_equals_mha_replicated(lib):
    rng = np.random.default_rng(15)
    B, Hq, D, T = 2, 5, 8, 9
    q, k1, v1 = _rand(rng, (B, Hq, D)), _rand(rng, (B, 1, T, D)), _rand(rng, (B, 1, T, D))
    L = np.array([9, 5], np.int32)
    mqa = _run(lib, q, k1, v1, L, 0.35)
    mha = _run(lib, q, np.repeat(k1, Hq, axis=1), np.repeat(v1, Hq, axis=1), L, 0.35)
    assert np.array_equal(mqa, mha)


def pin_gqa_is_independent_groups(lib):
    rng = np.random.default_rng(16)
    B, Hkv, M, D, T = 2, 3, 4, 8, 7
    Hq = Hkv * M
    q, k, v = _rand(rng, (B, Hq, D)), _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
    L = np.array([7, 2], np.int32)
    gqa = _run(lib, q, k, v, L, 0.35)
    for g in range(Hkv):
        part = _run(lib, np.ascontiguousarray(q[:, g * M:(g + 1) * M]),
                    np.ascontiguousarray(k[:, g:g + 1]), np.ascontiguousarray(v[:, g:g + 1]), L, 0.35)
        assert np.array_equal(gqa[:, g * M:(g + 1) * M], part), g


def pin_permutation_invariance(lib):
    rng = np.random.default_rng(17)
    B, Hq, Hkv, D, T = 2, 4, 2, 8, 10
    q, k, v = _rand(rng, (B, Hq, D)), _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
    L = np.array([10, 6], np.int32)
    base = _run(lib, q, k, v, L, 0.4)
    k2, v2 = k.copy(), v.copy()
    for b in range(B):
        perm = rng.permutation(L[b])
        k2[b, :, :L[b]] = k[b][:, perm]
        v2[b, :, :L[b]] = v[b][:, perm]
    assert np.allclose(_run(lib, q, k2, v2, L, 0.4), base, rtol=1e-12, atol=1e-13)


def pin_tail_never_read(lib):
    rng = np.random.default_rng(18)
    B, Hq, Hkv, D, T = 3, 4, 2, 8, 12
    q, k, v = _rand(rng, (B, Hq, D)), _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
    L = np.array([12, 5, 1], np.int32)
    base = _run(lib, q, k, v, L, 0.4)
    k2, v2 = k.copy(), v.copy()
    for b in range(B):
        k2[b, :, L[b]:] = np.nan
        v2[b, :, L[b]:] = np.inf
    got = _run(lib, q, k2, v2, L, 0.4)
    assert np.array_equal(got, base)
    # and a longer valid prefix does change the answer
    assert not np.allclose(_run(lib, q, k, v, np.array([12, 6, 1], np.int32), 0.4)[1], base[1])


def pin_key_shift_invariance(lib):
    rng = np.random.default_rng(19)
    B, Hq, Hkv, D, T = 2, 4, 1, 8, 9
    q, k, v = _rand(rng, (B, Hq, D)), _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
    L = np.array([9, 4], np.int32)
    u = _rand(rng, (1, 1, 1, D)) * np.float32(8)
    base = _run(lib, q, k, v, L, 0.3)
    shifted = _run(lib, q, (k + u).astype(np.float32), v, L, 0.3)
    # softmax ignores a per-head constant added to every score (up to the
    # fp32 rounding of k + u, which is why this is approximate)
    assert np.allclose(shifted, base, rtol=1e-5, atol=1e-6)


def pin_scale_moves_with_query(lib):
    rng = np.random.default_rng(20)
    B, Hq, Hkv, D, T = 2, 4, 2, 8, 9
    q, k, v = _rand(rng, (B, Hq, D)), _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
    L = np.array([9, 4], np.int32)
    a = _run(lib, q, k, v, L, 0.75)
    b = _run(lib, (q * np.float32(4)).astype(np.float32), k, v, L, 0.75 / 4)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)
    c = _run(lib, q, k, v, L, 0.75 * 3)
    assert not np.allclose(a, c, rtol=1e-3)


def pin_mpmath_bruteforce(lib):
    import mpmath
    mpmath.mp.dps = 50
    rng = np.random.default_rng(21)
    for trial in range(6):
        B, Hkv = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        M = int(rng.integers(1, 3))
        Hq, D, T = Hkv * M, int(rng.integers(1, 5)), int(rng.integers(1, 5))
        q, k, v = _rand(rng, (B, Hq, D)), _rand(rng, (B, Hkv, T, D)), _rand(rng, (B, Hkv, T, D))
        L = rng.integers(0, T + 1, size=B).astype(np.int32)
        scale = float(rng.uniform(0.1, 2.0))
        dtype = oracle.F32 if trial % 2 == 0 else oracle.BF16
        if dtype == oracle.BF16:
            # bf16-exact values: keep 8 significant bits
            q, k, v = [(np.asarray(x, np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
                       for x in (q, k, v)]
        got = _run(lib, q, k, v, L, scale, dtype)
        for b in range(B):
            for h in range(Hq):
                g, n = h // M, int(L[b])
                if n == 0:
                    assert np.all(got[b, h] == 0)
                    continue
                w = [mpmath.exp(mpmath.mpf(scale) * mpmath.fsum(
                    mpmath.mpf(float(q[b, h, j])) * mpmath.mpf(float(k[b, g, t, j])) for j in range(D)))
                    for t in range(n)]
                z = mpmath.fsum(w)
                for j in range(D):
                    ref = mpmath.fsum(w[t] * mpmath.mpf(float(v[b, g, t, j])) for t in range(n)) / z
                    assert abs(got[b, h, j] - float(ref)) <= 1e-13 * (1 + abs(float(ref))), (
                        trial, b, h, j, got[b, h, j], ref)


def pin_naive_recompute(lib):
    """Cached decoding == full causal attention recomputed from scratch."""
    rng = np.random.default_rng(22)
    T, E, Hq, Hkv, D = 9, 12, 4, 2, 8
    M = Hq // Hkv
    x = rng.standard_normal((T, E))
    Wq, Wk, Wv = (rng.standard_normal((E, n * D)) / math.sqrt(E) for n in (Hq, Hkv, Hkv))
    Q = (x @ Wq).reshape(T, Hq, D).astype(np.float32)
    K = (x @ Wk).reshape(T, Hkv, D).astype(np.float32)
    V = (x @ Wv).reshape(T, Hkv, D).astype(np.float32)
    scale = 1 / math.sqrt(D)

    # from scratch: full causal attention over the whole prefix at once
    full = np.zeros((T, Hq, D))
    for h in range(Hq):
        g = h // M
        S = scale * (Q[:, h].astype(np.float64) @ K[:, g].astype(np.float64).T)  # [T, T]
        S = np.where(np.tril(np.ones((T, T), bool)), S, -np.inf)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        full[:, h] = P @ V[:, g].astype(np.float64)

    # cached: start empty, append each token's K/V, attend its query
    kc = np.full((1, Hkv, T, D), np.nan, np.float32)
    vc = np.full((1, Hkv, T, D), np.nan, np.float32)
    L = np.zeros(1, np.int32)
    for i in range(T):
        kc, vc, L, ovf = oracle.append(kc, vc, L, K[i][None], V[i][None])
        assert not ovf.any() and L[0] == i + 1
        row = oracle.decode_attention(Q[i][None], kc, vc, L, scale, oracle.F32, lib=lib, threads=2)
        assert np.allclose(row[0], full[i], rtol=1e-12, atol=1e-13), i


PINS = [
    pin_golden, pin_single_token, pin_identical_keys_mean, pin_zero_query_mean, pin_argmax_limit,
    pin_mqa_equals_mha_replicated, pin_gqa_is_independent_groups, pin_permutation_invariance,
    pin_tail_never_read, pin_key_shift_invariance, pin_scale_moves_with_query,
    pin_mpmath_bruteforce, pin_naive_recompute,
]
