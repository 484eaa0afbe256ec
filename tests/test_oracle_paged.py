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
    distinct random page; unused pages hold NaN."""
    B, Hkv, T, D = contig.shape
    nb = T // P
    perm = rng.permutation(num_pages)[:B * nb].reshape(B, nb)
    pool = np.full((num_pages, Hkv, P, D), np.nan, dtype=contig.dtype)
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


# Planted mistakes in the paged oracle functions: each must fail a pin above.
PAGED_MUTANTS = {
    "offset_from_block": ("out[b, :, j * P:(j + 1) * P, :] = pages[page]",
                          "out[b, :, j * P:(j + 1) * P, :] = pages[page][:, ::-1]"),
    "table_transposed": ("page = int(bt[b, j])", "page = int(bt.T.ravel()[b * max_pages + j])"),
    "append_offset_is_block": ("k2[page, :, n[b] % P, :] = k_new[b]", "k2[page, :, n[b] // P, :] = k_new[b]"),
    "append_page_from_slot": ("page = int(bt[b, n[b] // P])", "page = int(bt[b, n[b] % bt.shape[1]])"),
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
