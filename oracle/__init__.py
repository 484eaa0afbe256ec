"""CPU oracle for decode attention over a KV cache (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and this
package never imports the GPU library: the two share nothing but the seeded
input generators, which hold none of the method's arithmetic.

* ``decode_attention`` wraps the fp64 C implementation in ``oracle.c``
  (definition written out: scores over the valid prefix, max-subtracted
  softmax over the sequence axis, weighted sum of values).
* ``append`` is the KV-cache append written out with numpy: write the new
  token's key and value at index ``lengths[b]`` of every KV head of sequence
  ``b`` and advance the length; a full sequence is left unchanged and
  reported.  Source: "All About Transformer Inference", section
  "Transformer inference basics" (generation appends the new token's
  key/value projections to the cache) and section "Implementation: JetStream"
  (generate appends the single-token KV cache to the decode state).

* ``gather_pages`` turns a paged cache back into the contiguous one it
  stands for: block j of sequence b (tokens j*P .. j*P+P-1) is page
  ``block_table[b, j]`` of the pool, token by token.  ``append_paged`` is the
  append on such a cache (the slot's page found the same way), and
  ``decode_attention_paged`` attends over the gathered cache.  Source: "All
  About Transformer Inference", section on tricks for generation
  throughput (paged attention: the KV cache kept in pages addressed through
  a table, so a batch holds only the memory it needs).

Parity status: every function is pinned by ``tests/test_oracle_pins.py``
and ``tests/test_oracle_paged.py``
(closed forms, exact hand-worked fixture, high-precision brute force,
invariants, naive full-prefix recomputation) and by
``tests/test_oracle_mutants.py`` (planted mistakes must fail a pin).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32 = 0
BF16 = 1


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the C oracle with gcc (plain -O2, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-pthread", src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str | None = None):
    """Load (building first if absent) an oracle shared library."""
    global _lib
    if path is None:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build()
        path = _LIB_PATH
    lib = ctypes.CDLL(path)
    fn = lib.oracle_decode_attention
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int] * 6 + [ctypes.c_void_p] * 4 + [
        ctypes.c_double, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
    if path == _LIB_PATH:
        _lib = lib
    return lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _as_bits(a: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F32:
        assert a.dtype == np.float32, a.dtype
    else:
        assert a.dtype == np.uint16, "bf16 arrays are passed as raw uint16 bit patterns"
    return np.ascontiguousarray(a)


def decode_attention(q, k_cache, v_cache, lengths, scale, dtype, rows=None,
                     threads=None, lib=None) -> np.ndarray:
    """fp64 decode attention.

    q: [B, Hq, D]; k_cache, v_cache: [B, Hkv, T_cap, D]; lengths: [B] int32.
    Arrays are float32 (dtype=F32) or raw bf16 bits as uint16 (dtype=BF16).
    rows: optional list of flattened (b*Hq + h) rows; returns [len(rows), D]
    in that order, else [B, Hq, D].
    """
    lib = lib or load()
    q = _as_bits(q, dtype)
    k_cache = _as_bits(k_cache, dtype)
    v_cache = _as_bits(v_cache, dtype)
    lengths = np.ascontiguousarray(lengths, dtype=np.int32)
    B, Hq, D = q.shape
    Bk, Hkv, T_cap, Dk = k_cache.shape
    assert Bk == B and Dk == D and v_cache.shape == k_cache.shape and lengths.shape == (B,)
    if rows is None:
        n_rows = B * Hq
        rows_arr = None
        out = np.zeros((B, Hq, D), dtype=np.float64)
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int32)
        n_rows = rows_arr.size
        out = np.zeros((n_rows, D), dtype=np.float64)
    rc = lib.oracle_decode_attention(
        B, Hq, Hkv, D, T_cap, dtype,
        q.ctypes.data, k_cache.ctypes.data, v_cache.ctypes.data, lengths.ctypes.data,
        float(scale), rows_arr.ctypes.data if rows_arr is not None else None, n_rows,
        out.ctypes.data, threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_decode_attention rejected its arguments (code {rc})")
    return out


def append(k_cache, v_cache, lengths, k_new, v_new):
    """KV-cache append, bit for bit.

    k_cache, v_cache: [B, Hkv, T_cap, D] (any dtype; copied, not modified);
    lengths: [B]; k_new, v_new: [B, Hkv, D].  Returns (k', v', lengths',
    overflow) where a sequence with lengths[b] == T_cap is left unchanged and
    flagged in ``overflow`` (bool [B]).
    """
    k2 = np.array(k_cache, copy=True)
    v2 = np.array(v_cache, copy=True)
    n = np.array(lengths, dtype=np.int64, copy=True)
    T_cap = k2.shape[2]
    overflow = np.zeros(n.shape, dtype=bool)
    for b in range(k2.shape[0]):
        if n[b] >= T_cap:
            overflow[b] = True
            continue
        k2[b, :, n[b], :] = k_new[b]
        v2[b, :, n[b], :] = v_new[b]
        n[b] += 1
    return k2, v2, n.astype(np.int32), overflow


def gather_pages(pages, block_table):
    """Contiguous cache [B, Hkv, max_pages * P, D] of a paged pool
    [num_pages, Hkv, P, D] under ``block_table`` [B, max_pages]: token t of
    sequence b is ``pages[block_table[b, t // P], :, t % P, :]``.  A block
    whose entry is not a page of the pool is filled with NaN (such blocks
    must lie past the sequence's length, where nothing is read)."""
    pages = np.asarray(pages)
    bt = np.asarray(block_table)
    num_pages, Hkv, P, D = pages.shape
    B, max_pages = bt.shape
    if pages.dtype.kind == "f":
        nan = np.full((Hkv, P, D), np.nan, dtype=pages.dtype)
    elif pages.dtype == np.uint16:  # bf16 bit patterns: quiet NaN
        nan = np.full((Hkv, P, D), 0x7FC0, dtype=np.uint16)
    else:
        nan = np.zeros((Hkv, P, D), dtype=pages.dtype)
    out = np.empty((B, Hkv, max_pages * P, D), dtype=pages.dtype)
    for b in range(B):
        for j in range(max_pages):
            page = int(bt[b, j])
            out[b, :, j * P:(j + 1) * P, :] = pages[page] if 0 <= page < num_pages else nan
    return out


def append_paged(k_pages, v_pages, block_table, lengths, k_new, v_new):
    """The append on a paged cache, bit for bit: slot n = lengths[b] of
    sequence b is offset n % P of page block_table[b, n // P].  Returns
    (k_pages', v_pages', lengths', overflow) like ``append``; the capacity
    is max_pages * P."""
    k2 = np.array(k_pages, copy=True)
    v2 = np.array(v_pages, copy=True)
    bt = np.asarray(block_table)
    n = np.array(lengths, dtype=np.int64, copy=True)
    P = k2.shape[2]
    cap = bt.shape[1] * P
    overflow = np.zeros(n.shape, dtype=bool)
    for b in range(bt.shape[0]):
        if n[b] >= cap:
            overflow[b] = True
            continue
        page = int(bt[b, n[b] // P])
        k2[page, :, n[b] % P, :] = k_new[b]
        v2[page, :, n[b] % P, :] = v_new[b]
        n[b] += 1
    return k2, v2, n.astype(np.int32), overflow


def decode_attention_paged(q, k_pages, v_pages, block_table, lengths, scale, dtype, **kw):
    """``decode_attention`` over the contiguous caches a paged pool stands for."""
    return decode_attention(q, gather_pages(k_pages, block_table), gather_pages(v_pages, block_table),
                            lengths, scale, dtype, **kw)
