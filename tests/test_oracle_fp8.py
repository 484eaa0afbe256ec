"""Pins of the fp8 (OCP E4M3, per-token power-of-two scale) cache oracle.

The decode is checked against values written out from the format's
definition; rounding against brute force over every finite code (nearest,
ties to the even code); the per-row exponent against its defining
inequality; the append against a hand-worked case.  Planted mistakes in
the oracle's fp8 functions must each fail one of these pins.
"""
import inspect
import types

import numpy as np
import pytest

import oracle

# code -> value from the format definition (1 sign, 4 exponent bits with
# bias 7, 3 mantissa bits; subnormals at exponent field 0; S.1111.111 NaN)
KNOWN = {
    0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
    0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x70: 128.0, 0x77: 240.0,
    0x78: 256.0, 0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xBC: -1.5, 0xFE: -448.0,
}


def test_decode_known_values():
    for code, v in KNOWN.items():
        got = oracle.e4m3_value(code)
        assert got == v and np.signbit(got) == np.signbit(v), (hex(code), got, v)
    assert np.isnan(oracle.e4m3_value(0x7F)) and np.isnan(oracle.e4m3_value(0xFF))


def test_decode_table_shape():
    t = oracle.E4M3_TABLE
    assert np.sum(np.isnan(t)) == 2
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0) and pos[-1] == 448.0      # increasing, max 448
    assert np.array_equal(t[0x80:0xFF], -pos)                   # sign symmetric


def _nearest_brute(y):
    finite = [c for c in range(256) if not np.isnan(oracle.E4M3_TABLE[c])]
    vals = np.array([oracle.E4M3_TABLE[c] for c in finite])
    out = []
    for x in np.ravel(y):
        d = np.abs(vals - x)
        best = [finite[i] for i in np.flatnonzero(d == d.min())]
        # same value twice only for +0/-0: take the sign of x
        vb = {oracle.E4M3_TABLE[c] for c in best}
        if len(vb) > 1:  # a true tie between two values: even mantissa
            best = [c for c in best if c % 2 == 0]
        best = [c for c in best if (c >= 0x80) == bool(np.signbit(x))] or best
        out.append(best[0])
    return np.array(out, dtype=np.uint8).reshape(np.shape(y))


def test_rounding_is_nearest_ties_to_even():
    rng = np.random.default_rng(1)
    y = np.concatenate([rng.uniform(-448, 448, 3000), rng.uniform(-2, 2, 3000),
                        rng.uniform(-2 ** -6, 2 ** -6, 1000)])
    # exact midpoints between neighbouring codes
    pos = oracle.E4M3_TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    y = np.concatenate([y, mids, -mids, [0.0, -0.0, 448.0, -448.0]])
    got = oracle._round_to_e4m3(y)
    assert np.array_equal(got, _nearest_brute(y))
    # hand-picked ties: 1 + 1/16 -> 1.0 (0x38), 1 + 3/16 -> 1.25 (0x3A)
    assert oracle._round_to_e4m3(np.array([1.0625, 1.1875, -1.0625])).tolist() == [0x38, 0x3A, 0xB8]


def test_quantize_hand_worked():
    codes, e = oracle.quantize_rows(np.array([[1.0, -0.5, 448.0, 0.0], [0.0, 0.0, 0.0, 0.0],
                                              [449.0, 0.0, 0.0, -1.0], [1.0, 0.0, 0.0, 0.0]]))
    assert e.tolist() == [0, 0, 1, -8]
    assert codes[0].tolist() == [0x38, 0xB0, 0x7E, 0x00]
    assert codes[1].tolist() == [0, 0, 0, 0]
    # amax 449 > 448: e = 1, and 224.5 rounds to 224 (0x76), -0.5 is 0xB0
    assert codes[2].tolist() == [0x76, 0x00, 0x00, 0xB0]
    assert codes[3].tolist() == [0x78, 0x00, 0x00, 0x00]  # 1 * 2^8 = 256


def test_quantize_exponent_is_minimal_and_error_bounded():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((500, 64)) * np.exp2(rng.integers(-20, 20, (500, 1)))
    codes, e = oracle.quantize_rows(x)
    amax = np.abs(x).max(axis=1)
    e = e.astype(np.float64)
    assert np.all(amax <= 448 * np.exp2(e)) and np.all(amax > 448 * np.exp2(e - 1))
    deq = oracle.dequantize(codes, e.astype(np.int8))
    # E4M3 keeps 3 mantissa bits: relative error <= 2^-4 on normals, and an
    # absolute error <= half the subnormal step 2^-10 * 2^e elsewhere
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * np.exp2(e)[:, None])
    assert np.all(err <= bound)


BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
BF16_MIN_NORMAL = 2.0 ** -126


def test_exponent_range_keeps_values_bf16_normal():
    """The stored exponent range is the reading that every code * 2^e is
    zero or a finite normal bf16 number, and it is the widest such range:
    one step further down the smallest code leaves bf16's normal range, one
    step up the largest code exceeds bf16's largest value."""
    vals = np.abs(oracle.E4M3_TABLE[np.isfinite(oracle.E4M3_TABLE)])
    nz = vals[vals > 0]
    for e in (oracle.E4M3_EXP_MIN, oracle.E4M3_EXP_MAX):
        scaled = nz * 2.0 ** e
        assert np.all(scaled >= BF16_MIN_NORMAL) and np.all(scaled <= BF16_MAX), e
    assert nz.min() * 2.0 ** (oracle.E4M3_EXP_MIN - 1) < BF16_MIN_NORMAL
    assert nz.max() * 2.0 ** (oracle.E4M3_EXP_MAX + 1) > BF16_MAX


def test_quantize_clamps_to_exponent_range():
    """Rows whose exponent falls outside the stored range: a tiny row takes
    the lowest exponent and rounds what lies below half the smallest code
    to zero (a tie goes to the even code 0); a huge row takes the highest
    and saturates at 448."""
    tiny = [2.0 ** -120, 2.0 ** -126, 2.0 ** -128, -(2.0 ** -127)]
    huge = [1.9 * 2.0 ** 127, -1.9 * 2.0 ** 127, 2.0 ** 119, 0.0]
    codes, e = oracle.quantize_rows(np.array([tiny, huge]))
    assert e.tolist() == [-117, 119]
    # 2^-120 * 2^117 = 2^-3 (0x20); 2^-9 is the smallest subnormal (0x01);
    # 2^-11 rounds to 0; -2^-10 is halfway between 0 and 2^-9: even code, signed
    assert codes[0].tolist() == [0x20, 0x01, 0x00, 0x80]
    assert codes[1].tolist() == [0x7E, 0xFE, 0x38, 0x00]


def test_append_fp8_hand_worked():
    B, Hkv, T, D = 2, 1, 3, 4
    kc = np.zeros((B, Hkv, T, D), np.uint8)
    ke = np.zeros((B, Hkv, T), np.int8)
    k_new = np.array([[[2.0, 0.0, -1.0, 0.25]], [[0.0, 0.0, 0.0, 0.0]]])
    kc2, ke2, vc2, ve2, L, of = oracle.append_fp8(kc, ke, kc, ke, np.array([1, 3]), k_new, k_new)
    # row 0: amax 2 = 1.0 * 2^1 -> e = 1 - 8 = -7; 2 * 2^7 = 256 (0x78), -1 -> -128 (0xF0), 0.25 -> 32 (0x60)
    assert ke2[0, 0, 1] == -7 and kc2[0, 0, 1].tolist() == [0x78, 0x00, 0xF0, 0x60]
    assert L.tolist() == [2, 3] and of.tolist() == [False, True]
    assert np.array_equal(kc2[1], kc[1]) and np.array_equal(kc2[0, 0, 0], kc[0, 0, 0])


def test_attention_over_dequantized_cache_brute_force():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, T, D = 2, 4, 2, 9, 8
    x = rng.standard_normal((2, B, Hkv, T, D))
    (kc, ke), (vc, ve) = oracle.quantize_rows(x[0]), oracle.quantize_rows(x[1])
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    L = np.array([9, 4], dtype=np.int32)
    got = oracle.decode_attention_fp8(q, kc, ke, vc, ve, L, 0.35)
    k, v = oracle.dequantize(kc, ke), oracle.dequantize(vc, ve)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            s = 0.35 * (k[b, g, :L[b]] @ q[b, h].astype(np.float64))
            p = np.exp(s - s.max())
            want = (p / p.sum()) @ v[b, g, :L[b]]
            assert np.allclose(got[b, h], want, rtol=1e-12, atol=1e-12)


FP8_MUTANTS = {
    "bias_8": ("* 2.0 ** (E - 7)", "* 2.0 ** (E - 8)"),
    "subnormal_scale": ("* (M / 8.0) * 2.0 ** -6", "* (M / 8.0) * 2.0 ** -7"),
    "ties_odd": ("np.where(_POS_CODES[lo] % 2 == 0, lo, hi)", "np.where(_POS_CODES[lo] % 2 == 1, lo, hi)"),
    "exponent_off_by_one": ("e[nz] = kk - 8 + (m > 1.75)", "e[nz] = kk - 7 + (m > 1.75)"),
    "exponent_threshold": ("e[nz] = kk - 8 + (m > 1.75)", "e[nz] = kk - 8 + (m >= 1.5)"),
    "scale_multiplied": ("y = x / np.exp2(e.astype(np.float64))[..., None]",
                         "y = np.clip(x * np.exp2(e.astype(np.float64))[..., None], -448, 448)"),
    "sign_dropped": ("return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)",
                     "return code.astype(np.uint8)"),
    "int8_exponent_range": ("E4M3_EXP_MIN = -117", "E4M3_EXP_MIN = -127"),
    "no_saturation": ("y = np.clip(y, -E4M3_MAX, E4M3_MAX)", "y = np.clip(y, -512.0, 512.0)"),
}


def _mutant(old, new):
    src = inspect.getsource(oracle)
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_fp8_mutant")
    mod.__file__ = oracle.__file__
    exec(compile(src.replace(old, new), "oracle_fp8_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_mutant_is_caught(name, monkeypatch):
    m = _mutant(*FP8_MUTANTS[name])
    pins = [test_decode_known_values, test_decode_table_shape, test_rounding_is_nearest_ties_to_even,
            test_quantize_hand_worked, test_quantize_exponent_is_minimal_and_error_bounded,
            test_exponent_range_keeps_values_bf16_normal, test_quantize_clamps_to_exponent_range,
            test_append_fp8_hand_worked]
    failed = []
    for pin in pins:
        with monkeypatch.context() as mp:
            for fn in ("e4m3_value", "E4M3_TABLE", "_POS_VALUES", "_POS_CODES", "_round_to_e4m3",
                       "quantize_rows", "dequantize", "append_fp8", "E4M3_EXP_MIN", "E4M3_EXP_MAX"):
                mp.setattr(oracle, fn, getattr(m, fn))
            try:
                pin()
            except (AssertionError, IndexError, ValueError):
                failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
