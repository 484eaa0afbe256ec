"""Pins of the paged-cache oracle (gather, append, attention) on the CPU.

The paged functions are pinned against a hand-worked fixture whose values
encode (page, KV head, offset), against a scatter written independently
here (gather must undo it exactly), and against the contiguous oracle
(appending and attending through pages must agree bit for bit with the
same operations on the gathered cache).
"""
import json
import os

import numpy as np
import pytest

import oracle
from multiquery_decode_attention_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "paged_gather_example.json")


def _fixture():
    with open(GOLDEN) as f:
        g = json.load(f)
    P, n, H = g["page_size"], g["num_pages"], g["num_kv_heads"]
    pool = np.zeros((n, H, P, 1), dtype=np.float64)
    for page in range(n):
        for h in range(H):
            for o in range(P):
                pool[page, h, o, 0] = 100 * page + 10 * h + o
    return g, pool, np.array(g["block_table"], dtype=np.int32)


def test_gather_hand_worked():
    g, pool, bt = _fixture()
    got = oracle.gather_pages(pool, bt)[..., 0]
    want = np.array([[[np.nan if x is None else x for x in row] for row in seq]
                     for seq in g["expected_contiguous"]["values"]], dtype=np.float64)
    assert got.shape == want.shape
    assert np.array_equal(got, want, equal_nan=True)


def test_append_paged_hand_worked():
    g, pool, bt = _fixture()
    a = g["append"]
    k_new = np.array(a["k_new"], dtype=np.float64)[..., None]
    k2, v2, L, overflow = oracle.append_paged(pool, pool, bt, np.array(a["lengths"]), k_new, k_new)
    assert np.array_equal(k2[..., 0], np.array(a["expected_pool"], dtype=np.float64))
    assert L.tolist() == a["expected_lengths"] and not overflow.any()


def _scatter(contig, P, num_pages, rng):
    """Independent inverse of the gather: every block of every sequence to a
    distinct random page; unused pages hold NaN (0x7F, the E4M3 NaN code,
    for uint8 codes)."""
    B, Hkv, T, D = contig.shape
    nb = T // P
    perm = rng.permutation(num_pages)[:B * nb].reshape(B, nb)
    pool = np.full((num_pages, Hkv, P, D), np.nan if contig.dtype.kind == "f" else 0x7F, dtype=contig.dtype)
    for b in range(B):
        for j in range(nb):
            for t in range(P):
                pool[perm[b, j], :, t, :] = contig[b, :, j * P + t, :]
    return pool, perm.astype(np.int32)


def test_gather_undoes_an_independent_scatter():
    rng = np.random.default_rng(5)
    contig = rng.standard_normal((3, 2, 12, 4))
    pool, bt = _scatter(contig, 4, 13, rng)
    assert np.array_equal(oracle.gather_pages(pool, bt), contig)


def test_input_generator_pages_gather_back():
    """inputs.make_paged (the shared seeded generator) lays pages out the
    way the oracle reads them."""
    case = inputs.make_case(3, 8, 2, 64, 96, [5, 40, 96], "bf16", seed=3)
    kp, vp, bt = inputs.make_paged(case.k_cache, case.v_cache, page_size=32, seed=4)
    k = inputs.host_array(case.k_cache)
    assert np.array_equal(oracle.gather_pages(inputs.host_array(kp), bt.numpy()), k)
    assert np.array_equal(oracle.gather_pages(inputs.host_array(vp), bt.numpy()),
                          inputs.host_array(case.v_cache))
    # every page is used at most once
    used = bt.numpy().ravel()
    assert len(np.unique(used)) == len(used)


@pytest.mark.parametrize("lengths", [[0, 7, 12], [12, 12, 3]])
def test_append_paged_commutes_with_gather(lengths):
    rng = np.random.default_rng(6)
    contig = rng.standard_normal((3, 2, 12, 4))
    pool, bt = _scatter(contig, 4, 11, rng)
    k_new = rng.standard_normal((3, 2, 4))
    k2, _, L2, of2 = oracle.append_paged(pool, pool, bt, np.array(lengths), k_new, k_new)
    c2, _, Lc, ofc = oracle.append(contig, contig, np.array(lengths), k_new, k_new)
    assert np.array_equal(oracle.gather_pages(k2, bt), c2)
    assert np.array_equal(L2, Lc) and np.array_equal(of2, ofc)


def test_paged_attention_equals_contiguous():
    rng = np.random.default_rng(7)
    B, Hq, Hkv, D, T, P = 3, 4, 2, 8, 16, 4
    k = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    L = np.array([16, 5, 9], dtype=np.int32)
    kp, bt = _scatter(k, P, 20, np.random.default_rng(8))
    vp, _ = _scatter(v, P, 20, np.random.default_rng(8))  # same permutation
    want = oracle.decode_attention(q, k, v, L, 0.3, oracle.F32)
    got = oracle.decode_attention_paged(q, kp, vp, bt, L, 0.3, oracle.F32)
    assert np.array_equal(got, want)


def _scatter_exps(contig, P, num_pages, perm):
    """Exponents [B, Hkv, T] into a pool [num_pages, Hkv, P] with the block
    permutation of ``_scatter`` (unused pages: 127)."""
    B, Hkv, T = contig.shape
    pool = np.full((num_pages, Hkv, P), 127, dtype=contig.dtype)
    for b in range(B):
        for j in range(T // P):
            for t in range(P):
                pool[perm[b, j], :, t] = contig[b, :, j * P + t]
    return pool


def _fp8_pools(lengths, seed):
    rng = np.random.default_rng(seed)
    B, Hkv, T, D, P = len(lengths), 2, 12, 8, 4
    codes = [rng.integers(0, 0x7E, (B, Hkv, T, D)).astype(np.uint8) for _ in range(2)]
    exps = [rng.integers(-9, -4, (B, Hkv, T)).astype(np.int8) for _ in range(2)]
    pools = []
    for c, e in zip(codes, exps):
        cp, bt = _scatter(c, P, 11, np.random.default_rng(seed + 1))  # same permutation for all four
        pools += [cp, _scatter_exps(e, P, 11, bt)]
    return codes, exps, pools, bt, rng


@pytest.mark.parametrize("lengths", [[0, 7, 12], [11, 3, 4], [9, 1, 6]])
def test_append_fp8_paged_commutes_with_gather(lengths):
    """Appending through the pages, then gathering, equals the contiguous
    fp8 append (codes, exponents, lengths and overflow bit for bit)."""
    (kc, vc), (ke, ve), (kcp, kep, vcp, vep), bt, rng = _fp8_pools(lengths, 12)
    k_new, v_new = rng.standard_normal((3, 2, 8)), rng.standard_normal((3, 2, 8)) * 40
    got = oracle.append_fp8_paged(kcp, kep, vcp, vep, bt, np.array(lengths), k_new, v_new)
    want = oracle.append_fp8(kc, ke, vc, ve, np.array(lengths), k_new, v_new)
    assert np.array_equal(oracle.gather_pages(got[0], bt), want[0])
    assert np.array_equal(oracle.gather_exponent_pages(got[1], bt), want[1])
    assert np.array_equal(oracle.gather_pages(got[2], bt), want[2])
    assert np.array_equal(oracle.gather_exponent_pages(got[3], bt), want[3])
    assert np.array_equal(got[4], want[4]) and np.array_equal(got[5], want[5])


def test_append_fp8_paged_hand_worked():
    """Slot 5 with 4-token pages is offset 1 of the sequence's second page."""
    kc = np.zeros((3, 1, 4, 4), np.uint8)
    ke = np.zeros((3, 1, 4), np.int8)
    bt = np.array([[2, 0]])
    k_new = np.array([[[2.0, 0.0, -1.0, 0.25]]])
    k2, e2, _, _, L, of = oracle.append_fp8_paged(kc, ke, kc, ke, bt, np.array([5]), k_new, k_new)
    assert L.tolist() == [6] and not of.any()
    # amax 2 -> e = -7; 2 -> 0x78, -1 -> 0xF0, 0.25 -> 0x60 (as in the contiguous hand-worked case)
    assert k2[0, 0, 1].tolist() == [0x78, 0x00, 0xF0, 0x60] and e2[0, 0, 1] == -7
    assert not k2[[1, 2]].any() and not k2[0, 0, [0, 2, 3]].any()


def test_fp8_paged_attention_equals_contiguous():
    (kc, vc), (ke, ve), (kcp, kep, vcp, vep), bt, rng = _fp8_pools([12, 5, 9], 13)
    q = rng.standard_normal((3, 4, 8)).astype(np.float32)
    L = np.array([12, 5, 9], dtype=np.int32)
    want = oracle.decode_attention_fp8(q, kc, ke, vc, ve, L, 0.3)
    got = oracle.decode_attention_fp8_paged(q, kcp, kep, vcp, vep, bt, L, 0.3)
    assert np.array_equal(got, want)


# Planted mistakes in the paged oracle functions: each must fail a pin above.
PAGED_MUTANTS = {
    "offset_from_block": ("out[b, :, j * P:(j + 1) * P, :] = pages[page]",
                          "out[b, :, j * P:(j + 1) * P, :] = pages[page][:, ::-1]"),
    "table_transposed": ("page = int(bt[b, j])", "page = int(bt.T.ravel()[b * max_pages + j])"),
    "append_offset_is_block": ("k2[page, :, n[b] % P, :] = k_new[b]", "k2[page, :, n[b] // P, :] = k_new[b]"),
    "append_page_from_slot": ("page = int(bt[b, n[b] // P])", "page = int(bt[b, n[b] % bt.shape[1]])"),
}
FP8_PAGED_MUTANTS = {
    "fp8_offset_is_block": ("page, off = int(bt[b, n[b] // P]), n[b] % P", "page, off = int(bt[b, n[b] // P]), n[b] // P"),
    "fp8_page_from_slot": ("page, off = int(bt[b, n[b] // P]), n[b] % P",
                           "page, off = int(bt[b, n[b] % bt.shape[1]]), n[b] % P"),
    "fp8_exponent_swapped": ("kc[page, :, off, :], ke[page, :, off] = qk[b], ek[b]",
                             "kc[page, :, off, :], ke[page, :, off] = qk[b], ev[b]"),
    "fp8_gather_exps_wrong_axis": ("return gather_pages(np.asarray(exp_pages)[..., None], block_table)[..., 0]",
                                   "return gather_pages(np.asarray(exp_pages)[..., ::-1, None], block_table)[..., 0]"),
}


def _mutated_module(old, new):
    import inspect
    import types
    src = inspect.getsource(oracle)
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = oracle.__file__
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(PAGED_MUTANTS))
def test_paged_mutant_is_caught(name, monkeypatch):
    mutant = _mutated_module(*PAGED_MUTANTS[name])
    pins = [test_gather_hand_worked, test_append_paged_hand_worked,
            test_gather_undoes_an_independent_scatter]
    failed = []
    for pin in pins:
        with monkeypatch.context() as m:
            m.setattr(oracle, "gather_pages", mutant.gather_pages)
            m.setattr(oracle, "append_paged", mutant.append_paged)
            try:
                pin()
            except (AssertionError, IndexError, ValueError):
                failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(FP8_PAGED_MUTANTS))
def test_fp8_paged_mutant_is_caught(name, monkeypatch):
    mutant = _mutated_module(*FP8_PAGED_MUTANTS[name])
    pins = [lambda: test_append_fp8_paged_commutes_with_gather([0, 7, 12]),
            lambda: test_append_fp8_paged_commutes_with_gather([11, 3, 4]),
            lambda: test_append_fp8_paged_commutes_with_gather([9, 1, 6]),
            test_append_fp8_paged_hand_worked, test_fp8_paged_attention_equals_contiguous]
    failed = 0
    for pin in pins:
        with monkeypatch.context() as m:
            for fn in ("append_fp8_paged", "gather_exponent_pages", "decode_attention_fp8_paged"):
                m.setattr(oracle, fn, getattr(mutant, fn))
            try:
                pin()
            except (AssertionError, IndexError, ValueError):
                failed += 1
    assert failed, f"mutant {name} passed every pin"
