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

* The fp8 cache: K and V stored as OCP FP8 E4M3 codes (1 sign, 4 exponent
  bits with bias 7, 3 mantissa bits; largest finite 448, codes 0x7F/0xFF are
  NaN, no infinities) with one power-of-two scale 2^e per (sequence, KV
  head, token).  ``e4m3_value`` decodes a code from that definition;
  ``quantize_rows`` picks, for each row, the smallest e with
  max|x| / 2^e <= 448 and rounds x / 2^e to the nearest code (ties to the
  even code); ``dequantize`` is code value * 2^e; ``append_fp8`` quantizes
  the new token into its slot; ``decode_attention_fp8`` attends over the
  dequantized cache.  Source: "All About Transformer Inference", section on
  tricks for generation throughput (quantizing the KV cache to int8, int4
  or fp8 saves memory bandwidth); "Efficiently Scaling Transformer
  Inference", section 3.6 (quantized storage, bf16 arithmetic for the
  products).  The pages fix no scale format: per-token power-of-two scales
  are this library's choice.

* Several new tokens per sequence (a speculative-verify step): ``append_multi``
  writes T_q new K/V rows at slots lengths[b] .. lengths[b]+T_q-1 (or none,
  when they do not fit), and ``decode_attention_multi`` lets query i of
  sequence b attend over the tokens before it and itself: the first
  n - a + min(i + 1, a) cached tokens, with n the length after the append
  and a the number of rows appended.  Source: "All About Transformer
  Inference", appendix on speculative sampling (the large model scores all
  drafted tokens in one pass, sharing the KV cache load) and section
  "Transformer inference basics" (a token attends to the tokens before it).

Parity status: every function is pinned by ``tests/test_oracle_pins.py``,
``tests/test_oracle_paged.py``, ``tests/test_oracle_fp8.py`` and
``tests/test_oracle_multi.py``
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
    """Load (building first if absent) an oracle shared library.
    KVD_ORACLE_LIBRARY may name another build of oracle.c (the sanitizer
    run of the CPU tests uses one)."""
    global _lib
    if path is None:
        if _lib is not None:
            return _lib
        other = os.environ.get("KVD_ORACLE_LIBRARY")
        if other:
            _lib = load(other)
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
    """Threads for the oracle: the CPUs this process may run on, or fewer
    when OMP_NUM_THREADS sets the host's share."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    try:
        share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    except ValueError:
        share = 0
    return max(1, min(n, share) if share > 0 else n)


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


# --- fp8 (OCP E4M3) cache ----------------------------------------------------

E4M3_MAX = 448.0
# Range of the stored power-of-two exponents.  The pages fix no scale format;
# this library's reading keeps every code * 2^e zero or a finite normal
# bfloat16 number: the smallest subnormal code 2^-9 times 2^-117 is 2^-126
# (the smallest normal bf16), and 448 * 2^119 = 1.75 * 2^127 is below the
# largest bf16.  An append clamps each row's exponent into it.
E4M3_EXP_MIN = -117
E4M3_EXP_MAX = 119


def e4m3_value(code: int) -> float:
    """Value of an OCP FP8 E4M3 code: (-1)^s * 2^(E-7) * (1 + M/8) for
    E >= 1, (-1)^s * 2^-6 * M/8 for E = 0; E = 15 with M = 7 is NaN."""
    s = -1.0 if code & 0x80 else 1.0
    E = (code >> 3) & 0xF
    M = code & 0x7
    if E == 0xF and M == 0x7:
        return float("nan")
    if E == 0:
        return s * (M / 8.0) * 2.0 ** -6
    return s * (1.0 + M / 8.0) * 2.0 ** (E - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# finite non-negative codes in increasing order of value (0x00 .. 0x7E)
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = E4M3_TABLE[:0x7F]


def _round_to_e4m3(y: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of each |y| <= 448 (ties to the code with an even
    mantissa), sign taken from y's sign bit (so -0.0 -> 0x80)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    assert np.all(a <= E4M3_MAX), "value outside the E4M3 range"
    # index of the first representable value >= a
    hi = np.searchsorted(_POS_VALUES, a, side="left")
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = (d_lo == d_hi) & (lo != hi)
    pick = np.where(tie, np.where(_POS_CODES[lo] % 2 == 0, lo, hi), pick)
    code = _POS_CODES[pick]
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def quantize_rows(x):
    """Quantize each row (last axis) of x to (codes uint8, exponent int8).

    e is the smallest integer with max|x| <= 448 * 2^e, clamped to
    [E4M3_EXP_MIN, E4M3_EXP_MAX] (0 for an all-zero row); codes are x / 2^e
    rounded to E4M3, saturated at +-448 when e was clamped at the top.  x
    must be finite.
    """
    x = np.asarray(x, dtype=np.float64)
    amax = np.max(np.abs(x), axis=-1)
    assert np.all(np.isfinite(amax)), "non-finite value to quantize"
    e = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    # smallest e with amax <= 448 * 2^e, from amax = f * 2^k, f in [0.5, 1)
    f, k = np.frexp(amax[nz])
    m, kk = 2.0 * f, k - 1                 # amax = m * 2^kk, m in [1, 2)
    e[nz] = kk - 8 + (m > 1.75)
    e = np.clip(e, E4M3_EXP_MIN, E4M3_EXP_MAX)
    y = x / np.exp2(e.astype(np.float64))[..., None]
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)  # only reached when e was clamped
    return _round_to_e4m3(y), e.astype(np.int8)


def dequantize(codes, exps):
    """codes [..., D] uint8 and exps [...] int8 -> float64 values."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.int64)] * np.exp2(np.asarray(exps, dtype=np.float64))[..., None]


def append_fp8(k_codes, k_exps, v_codes, v_exps, lengths, k_new, v_new):
    """The append on an fp8 cache: the new token's K and V rows (any float
    array [B, Hkv, D]) are quantized per (sequence, KV head) into slot
    lengths[b].  Returns (k_codes', k_exps', v_codes', v_exps', lengths',
    overflow)."""
    kc, ke = np.array(k_codes, copy=True), np.array(k_exps, copy=True)
    vc, ve = np.array(v_codes, copy=True), np.array(v_exps, copy=True)
    n = np.array(lengths, dtype=np.int64, copy=True)
    T_cap = kc.shape[2]
    qk, ek = quantize_rows(k_new)
    qv, ev = quantize_rows(v_new)
    overflow = np.zeros(n.shape, dtype=bool)
    for b in range(kc.shape[0]):
        if n[b] >= T_cap:
            overflow[b] = True
            continue
        kc[b, :, n[b], :], ke[b, :, n[b]] = qk[b], ek[b]
        vc[b, :, n[b], :], ve[b, :, n[b]] = qv[b], ev[b]
        n[b] += 1
    return kc, ke, vc, ve, n.astype(np.int32), overflow


def decode_attention_fp8(q, k_codes, k_exps, v_codes, v_exps, lengths, scale, **kw):
    """Decode attention over the dequantized fp8 cache.  q is a float32
    array (a bf16 query widened exactly); the dequantized values are exact
    in float32 for the exponent range the tests use."""
    k = dequantize(k_codes, k_exps)
    v = dequantize(v_codes, v_exps)
    L = np.asarray(lengths)
    # slots past the lengths are never read; keep their values finite here
    k32, v32 = k.astype(np.float32), v.astype(np.float32)
    assert np.array_equal(k32.astype(np.float64)[np.isfinite(k)], k[np.isfinite(k)])
    return decode_attention(np.asarray(q, dtype=np.float32), k32, v32, L, scale, F32, **kw)


def append_fp8_paged(kc_pages, ke_pages, vc_pages, ve_pages, block_table, lengths, k_new, v_new):
    """``append_fp8`` on page pools: code pools [num_pages, Hkv, P, D] uint8
    and exponent pools [num_pages, Hkv, P] int8; slot n = lengths[b] of
    sequence b is offset n % P of page block_table[b, n // P] (as in
    ``append_paged``), and the capacity is max_pages * P."""
    kc, ke = np.array(kc_pages, copy=True), np.array(ke_pages, copy=True)
    vc, ve = np.array(vc_pages, copy=True), np.array(ve_pages, copy=True)
    bt = np.asarray(block_table)
    n = np.array(lengths, dtype=np.int64, copy=True)
    P = kc.shape[2]
    cap = bt.shape[1] * P
    qk, ek = quantize_rows(k_new)
    qv, ev = quantize_rows(v_new)
    overflow = np.zeros(n.shape, dtype=bool)
    for b in range(bt.shape[0]):
        if n[b] >= cap:
            overflow[b] = True
            continue
        page, off = int(bt[b, n[b] // P]), n[b] % P
        kc[page, :, off, :], ke[page, :, off] = qk[b], ek[b]
        vc[page, :, off, :], ve[page, :, off] = qv[b], ev[b]
        n[b] += 1
    return kc, ke, vc, ve, n.astype(np.int32), overflow


def gather_exponent_pages(exp_pages, block_table):
    """Contiguous exponents [B, Hkv, max_pages * P] of an exponent pool
    [num_pages, Hkv, P] (``gather_pages`` on a trailing axis of one)."""
    return gather_pages(np.asarray(exp_pages)[..., None], block_table)[..., 0]


def decode_attention_fp8_paged(q, kc_pages, ke_pages, vc_pages, ve_pages, block_table, lengths, scale, **kw):
    """``decode_attention_fp8`` over the contiguous cache the pools stand for."""
    g = lambda x: gather_pages(x, block_table)
    return decode_attention_fp8(q, g(kc_pages), gather_exponent_pages(ke_pages, block_table), g(vc_pages),
                                gather_exponent_pages(ve_pages, block_table), lengths, scale, **kw)


# --- several new tokens per sequence -----------------------------------------

def append_multi(k_cache, v_cache, lengths, k_new, v_new):
    """Append T_q tokens per sequence: k_new, v_new [B, Hkv, T_q, D] go to
    slots lengths[b] .. lengths[b] + T_q - 1 in order.  A sequence they do not
    fit is left unchanged and flagged.  Returns (k', v', lengths', appended)
    with appended[b] = T_q or 0."""
    k2 = np.array(k_cache, copy=True)
    v2 = np.array(v_cache, copy=True)
    n = np.array(lengths, dtype=np.int64, copy=True)
    T_cap = k2.shape[2]
    T_q = np.asarray(k_new).shape[2]
    appended = np.zeros(n.shape, dtype=np.int32)
    for b in range(k2.shape[0]):
        if n[b] < 0 or n[b] + T_q > T_cap:
            continue
        for i in range(T_q):
            k2[b, :, n[b] + i, :] = k_new[b, :, i]
            v2[b, :, n[b] + i, :] = v_new[b, :, i]
        n[b] += T_q
        appended[b] = T_q
    return k2, v2, n.astype(np.int32), appended


def decode_attention_multi(q, k_cache, v_cache, lengths, appended, scale, dtype, **kw):
    """q [B, Hq, T_q, D]; lengths after the append, appended [B] rows added.
    Query i of sequence b attends over its first
    lengths[b] - appended[b] + min(i + 1, appended[b]) tokens.  Returns
    [B, Hq, T_q, D]."""
    q = np.asarray(q)
    B, Hq, T_q, D = q.shape
    L = np.asarray(lengths, dtype=np.int64)
    a = np.asarray(appended, dtype=np.int64)
    out = np.empty((B, Hq, T_q, D), dtype=np.float64)
    for i in range(T_q):
        Li = (L - a + np.minimum(i + 1, a)).astype(np.int32)
        out[:, :, i, :] = decode_attention(np.ascontiguousarray(q[:, :, i, :]), k_cache, v_cache, Li, scale,
                                           dtype, **kw)
    return out


# --- fp8 cache, several new tokens per sequence -------------------------------

def append_fp8_multi(k_codes, k_exps, v_codes, v_exps, lengths, k_new, v_new):
    """``append_multi`` on an fp8 cache: every new row of k_new, v_new
    [B, Hkv, T_q, D] (any float array) is quantized (``quantize_rows``) into
    slots lengths[b] .. lengths[b] + T_q - 1; a sequence they do not fit is
    left unchanged.  Returns (k_codes', k_exps', v_codes', v_exps', lengths',
    appended) with appended[b] = T_q or 0."""
    kc, ke = np.array(k_codes, copy=True), np.array(k_exps, copy=True)
    vc, ve = np.array(v_codes, copy=True), np.array(v_exps, copy=True)
    n = np.array(lengths, dtype=np.int64, copy=True)
    T_cap = kc.shape[2]
    T_q = np.asarray(k_new).shape[2]
    qk, ek = quantize_rows(k_new)
    qv, ev = quantize_rows(v_new)
    appended = np.zeros(n.shape, dtype=np.int32)
    for b in range(kc.shape[0]):
        if n[b] < 0 or T_cap - n[b] < T_q:  # no room for all T_q rows
            continue
        for i in range(T_q):
            kc[b, :, n[b] + i, :], ke[b, :, n[b] + i] = qk[b, :, i], ek[b, :, i]
            vc[b, :, n[b] + i, :], ve[b, :, n[b] + i] = qv[b, :, i], ev[b, :, i]
        n[b] += T_q
        appended[b] = T_q
    return kc, ke, vc, ve, n.astype(np.int32), appended


def decode_attention_fp8_multi(q, k_codes, k_exps, v_codes, v_exps, lengths, appended, scale, **kw):
    """``decode_attention_multi`` over the dequantized fp8 cache; q
    [B, Hq, T_q, D] float32 (bf16 queries widened exactly)."""
    k = dequantize(k_codes, k_exps).astype(np.float32)
    v = dequantize(v_codes, v_exps).astype(np.float32)
    return decode_attention_multi(np.asarray(q, dtype=np.float32), k, v, lengths, appended, scale, F32, **kw)
