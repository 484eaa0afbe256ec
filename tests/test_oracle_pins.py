"""The CPU oracle against its pins (no GPU)."""
import numpy as np
import pytest

import oracle
from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_append_writes_slot_and_advances():
    """The append oracle: slot lengths[b] of every KV head takes the new
    token, nothing else changes, lengths advance; a full sequence is left
    as is and flagged."""
    rng = np.random.default_rng(30)
    B, Hkv, T, D = 3, 2, 4, 8
    k = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    L = np.array([0, 2, 4], np.int32)
    kn = rng.standard_normal((B, Hkv, D)).astype(np.float32)
    vn = rng.standard_normal((B, Hkv, D)).astype(np.float32)
    k2, v2, L2, ovf = oracle.append(k, v, L, kn, vn)
    assert L2.tolist() == [1, 3, 4] and ovf.tolist() == [False, False, True]
    for b, n in enumerate(L):
        for t in range(T):
            if t == n and n < T:
                assert np.array_equal(k2[b, :, t], kn[b]) and np.array_equal(v2[b, :, t], vn[b])
            else:
                assert np.array_equal(k2[b, :, t], k[b, :, t]) and np.array_equal(v2[b, :, t], v[b, :, t])
    # bit patterns survive (bf16 as raw uint16, including NaN payloads)
    kb = rng.integers(0, 2**16, size=(1, 1, 2, 4), dtype=np.uint16)
    nb = np.array([[[0x7FC1, 0xFF80, 0x0001, 0x8000]]], np.uint16)
    k3, _, L3, _ = oracle.append(kb, kb, np.array([1], np.int32), nb, nb)
    assert k3[0, 0, 1].tobytes() == nb[0, 0].tobytes() and L3[0] == 2


def test_oracle_rejects_bad_lengths(oracle_lib):
    q = np.zeros((1, 1, 4), np.float32)
    k = np.zeros((1, 1, 2, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.decode_attention(q, k, k, np.array([3], np.int32), 1.0, oracle.F32, lib=oracle_lib)
    with pytest.raises(ValueError):
        oracle.decode_attention(q, k, k, np.array([-1], np.int32), 1.0, oracle.F32, lib=oracle_lib)


def test_oracle_rows_subset_matches_full(oracle_lib):
    rng = np.random.default_rng(31)
    B, Hq, Hkv, D, T = 3, 6, 3, 16, 20
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    L = np.array([20, 7, 0], np.int32)
    full = oracle.decode_attention(q, k, v, L, 0.25, oracle.F32, lib=oracle_lib)
    rows = [17, 0, 5, 12, 9]
    sub = oracle.decode_attention(q, k, v, L, 0.25, oracle.F32, rows=rows, lib=oracle_lib)
    assert np.array_equal(sub, full.reshape(B * Hq, D)[rows])
