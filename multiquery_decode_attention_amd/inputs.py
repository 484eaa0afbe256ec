"""Seeded synthetic inputs for decode attention over a KV cache.

This module holds the workload recipes only -- shapes, value distributions,
length mixes and seeds -- and none of the attention arithmetic.  It is the one
module both the GPU path's tests/bench and the CPU oracle's callers share.

Workloads (shapes from the pages; the pages publish no dataset, so every
tensor is drawn from a seeded generator):

* ``tiny_mqa_f32``      -- fp32, B=1, Hq=8, Hkv=1, d=64; 128 cached tokens,
  one new token appended, then attended (129 keys).
* ``palm_mqa_bf16``     -- PaLM-540B-like multiquery layer: 48 query heads,
  d_head 256, one KV head, context 2048 ("Efficiently Scaling Transformer
  Inference", sections 3.3 and 4), batch 64.
* ``llama13b_mha_bf16`` -- LLaMA-2-13B-like multi-head layer: 40 heads of
  d 128, no sharing ("How to Parallelize a Transformer for Training", model
  table), batch 32, context 4096.
* ``ragged_gqa_bf16``   -- grouped-query with 8 KV heads ("All About
  Transformer Inference", GQA paragraph), 64 query heads of d 128, batch 128,
  per-sequence lengths uniform on [64, 8192] (continuous batching with ragged
  reads), keys scaled by 3 to sharpen the softmax.
* ``longctx_mqa_bf16``  -- 32x the 2048 context of the PaLM setting: B=8,
  T=65536, 48 query heads over one KV head of d 256.

Every draw is N(0, 1) in fp32, scaled where the recipe says so, then rounded
once to the cache dtype (round-to-nearest-even via ``Tensor.to``).  Lengths
are drawn on a CPU generator so they do not depend on the device.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

SEED_BASE = 20261202


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    D: int
    T: int                # attended length after the step's append (max for ragged)
    T_cap: int            # cache capacity
    ragged: tuple = ()    # (lo, hi) inclusive range of attended lengths, or ()
    k_scale: float = 1.0
    seed_index: int = 0

    @property
    def seed(self) -> int:
        return SEED_BASE + self.seed_index

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def scale(self) -> float:
        return float(self.D) ** -0.5


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_mqa_f32", "f32", 1, 8, 1, 64, 129, 160, seed_index=0),
        Workload("palm_mqa_bf16", "bf16", 64, 48, 1, 256, 2048, 2048, seed_index=1),
        Workload("llama13b_mha_bf16", "bf16", 32, 40, 40, 128, 4096, 4096, seed_index=2),
        Workload("ragged_gqa_bf16", "bf16", 128, 64, 8, 128, 8192, 8192, ragged=(64, 8192),
                 k_scale=3.0, seed_index=3),
        Workload("longctx_mqa_bf16", "bf16", 8, 48, 1, 256, 65536, 65536, seed_index=4),
    ]
}


@dataclasses.dataclass
class Case:
    """One decode step's inputs.

    lengths0 are the cached lengths BEFORE the step's append; after the
    append every sequence holds lengths0 + 1 tokens (the attended lengths).
    """
    q: torch.Tensor          # [B, Hq, D]
    k_cache: torch.Tensor    # [B, Hkv, T_cap, D]
    v_cache: torch.Tensor    # [B, Hkv, T_cap, D]
    lengths0: torch.Tensor   # [B] int32
    k_new: torch.Tensor      # [B, Hkv, D]
    v_new: torch.Tensor      # [B, Hkv, D]
    scale: float


def attended_lengths(w: Workload, B: Optional[int] = None) -> torch.Tensor:
    """Per-sequence attended lengths (after the append), int32 on the CPU."""
    B = w.B if B is None else B
    if w.ragged:
        g = torch.Generator(device="cpu").manual_seed(w.seed + 7919)
        lo, hi = w.ragged
        return torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    return torch.full((B,), w.T, dtype=torch.int32)


def _normal(shape, gen, device, dtype, k=1.0, chunk_elems=1 << 28):
    """N(0,1) draws in fp32, optionally scaled, rounded once to ``dtype``."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        x = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32)
        if k != 1.0:
            x.mul_(k)
        flat[s:e] = x.to(dtype)
    return out


def make_case(B, Hq, Hkv, D, T_cap, lengths_attended, dtype, seed, device="cpu",
              k_scale=1.0) -> Case:
    """Seeded case of arbitrary shape.  Cache rows at or beyond the attended
    length are filled with draws too (they must never be read)."""
    tdt = torch.float32 if dtype in ("f32", torch.float32) else torch.bfloat16
    lengths_attended = torch.as_tensor(lengths_attended, dtype=torch.int32).cpu()
    assert lengths_attended.shape == (B,)
    assert int(lengths_attended.min()) >= 1 and int(lengths_attended.max()) <= T_cap
    gen = torch.Generator(device=device).manual_seed(int(seed))
    q = _normal((B, Hq, D), gen, device, tdt)
    k_cache = _normal((B, Hkv, T_cap, D), gen, device, tdt, k=k_scale)
    v_cache = _normal((B, Hkv, T_cap, D), gen, device, tdt)
    k_new = _normal((B, Hkv, D), gen, device, tdt, k=k_scale)
    v_new = _normal((B, Hkv, D), gen, device, tdt)
    lengths0 = (lengths_attended - 1).to(torch.int32).to(device)
    return Case(q, k_cache, v_cache, lengths0, k_new, v_new, float(D) ** -0.5)


def make_workload_case(w: Workload, device="cpu", seed: Optional[int] = None,
                       B: Optional[int] = None) -> Case:
    """The named workload (optionally with a smaller batch for CPU tests)."""
    B = w.B if B is None else B
    return make_case(B, w.Hq, w.Hkv, w.D, w.T_cap, attended_lengths(w, B), w.dtype,
                     w.seed if seed is None else seed, device, k_scale=w.k_scale)


@dataclasses.dataclass
class MultiCase:
    """A step with T_q new tokens per sequence (drafted tokens to verify)."""
    q: torch.Tensor          # [B, Hq, T_q, D]
    k_cache: torch.Tensor    # [B, Hkv, T_cap, D]
    v_cache: torch.Tensor
    lengths0: torch.Tensor   # [B] int32, before the append
    k_new: torch.Tensor      # [B, Hkv, T_q, D]
    v_new: torch.Tensor
    scale: float


def make_multi_case(B, Hq, Hkv, D, T_cap, lengths0, T_q, dtype, seed, device="cpu") -> MultiCase:
    """Seeded case with T_q new tokens per sequence; lengths0 are the cached
    lengths before the step (they may leave no room, to test overflow)."""
    tdt = torch.float32 if dtype in ("f32", torch.float32) else torch.bfloat16
    gen = torch.Generator(device=device).manual_seed(int(seed))
    q = _normal((B, Hq, T_q, D), gen, device, tdt)
    k_cache = _normal((B, Hkv, T_cap, D), gen, device, tdt)
    v_cache = _normal((B, Hkv, T_cap, D), gen, device, tdt)
    k_new = _normal((B, Hkv, T_q, D), gen, device, tdt)
    v_new = _normal((B, Hkv, T_q, D), gen, device, tdt)
    lengths0 = torch.as_tensor(lengths0, dtype=torch.int32).to(device)
    return MultiCase(q, k_cache, v_cache, lengths0, k_new, v_new, float(D) ** -0.5)


@dataclasses.dataclass
class Fp8Case:
    """One decode step over an fp8 cache: E4M3 codes and per-row
    power-of-two exponents (value = code * 2^e); bf16 query and new rows."""
    q: torch.Tensor          # [B, Hq, D] bf16
    k_codes: torch.Tensor    # [B, Hkv, T_cap, D] uint8
    k_exp: torch.Tensor      # [B, Hkv, T_cap] int8
    v_codes: torch.Tensor
    v_exp: torch.Tensor
    lengths0: torch.Tensor   # [B] int32, before the step's append
    k_new: torch.Tensor      # [B, Hkv, D] bf16
    v_new: torch.Tensor
    scale: float


def _e4m3_codes(shape, gen, device):
    """Random finite E4M3 codes: uniform sign, exponent field 0..15 and
    mantissa, so every finite code -- the subnormals of field 0 and zero
    included -- is drawn; the NaN pattern S.1111.111 is mapped to
    S.1111.110."""
    S = torch.randint(0, 2, shape, generator=gen, device=device, dtype=torch.int32)
    E = torch.randint(0, 16, shape, generator=gen, device=device, dtype=torch.int32)
    M = torch.randint(0, 8, shape, generator=gen, device=device, dtype=torch.int32)
    M = torch.where((E == 15) & (M == 7), torch.full_like(M, 6), M)
    return ((S << 7) | (E << 3) | M).to(torch.uint8)


# Stored row exponents of the fp8 cache format: [-117, 119].
FP8_EXP_MIN, FP8_EXP_MAX = -117, 119


def _row_exponents(shape, gen, device, lo, hi, wide_lo, wide_hi):
    """Per-row exponents: 7 of 8 rows uniform on [lo, hi], the rest uniform
    on [wide_lo, wide_hi]."""
    base = torch.randint(lo, hi + 1, shape, generator=gen, device=device, dtype=torch.int32)
    wide = torch.randint(wide_lo, wide_hi + 1, shape, generator=gen, device=device, dtype=torch.int32)
    pick = torch.randint(0, 8, shape, generator=gen, device=device, dtype=torch.int32) == 0
    return torch.where(pick, wide, base).to(torch.int8)


def make_fp8_case(B, Hq, Hkv, D, T_cap, lengths_attended, seed, device="cpu",
                  new_tokens: Optional[int] = None, k_exp_value: Optional[int] = None,
                  v_exp_value: Optional[int] = None) -> Fp8Case:
    """Seeded fp8-cache case: the cache is drawn directly as codes and
    exponents (no quantization here: that is the method's own step, done by
    the append under test and by the oracle); q and the new rows are N(0,1)
    rounded to bf16.  Codes cover every finite E4M3 code.  Row exponents:
    keys mostly in [-12, -4] with one row in eight at the bottom of the
    stored range, [-117, -100] (keys that score about 0); values mostly in
    [-12, -4] with one row in eight anywhere in [-117, 32] (32 keeps the
    fp32 sums of weighted values far from overflow at any length).
    ``k_exp_value`` / ``v_exp_value`` instead give every row that exponent.
    With ``new_tokens`` T the step appends T rows per sequence (k_new, v_new
    [B, Hkv, T, D], q [B, Hq, T, D]) and the lengths before it are
    lengths_attended - T."""
    T = 1 if new_tokens is None else int(new_tokens)
    extra = () if new_tokens is None else (T,)
    lengths_attended = torch.as_tensor(lengths_attended, dtype=torch.int32).cpu()
    assert lengths_attended.shape == (B,)
    assert int(lengths_attended.min()) >= 1 and int(lengths_attended.max()) <= T_cap
    gen = torch.Generator(device=device).manual_seed(int(seed))
    q = _normal((B, Hq) + extra + (D,), gen, device, torch.bfloat16)
    k_codes = _e4m3_codes((B, Hkv, T_cap, D), gen, device)
    v_codes = _e4m3_codes((B, Hkv, T_cap, D), gen, device)
    k_exp = _row_exponents((B, Hkv, T_cap), gen, device, -12, -4, FP8_EXP_MIN, -100)
    v_exp = _row_exponents((B, Hkv, T_cap), gen, device, -12, -4, FP8_EXP_MIN, 32)
    if k_exp_value is not None:
        k_exp = torch.full_like(k_exp, int(k_exp_value))
    if v_exp_value is not None:
        v_exp = torch.full_like(v_exp, int(v_exp_value))
    k_new = _normal((B, Hkv) + extra + (D,), gen, device, torch.bfloat16)
    v_new = _normal((B, Hkv) + extra + (D,), gen, device, torch.bfloat16)
    assert int(lengths_attended.min()) >= T
    lengths0 = (lengths_attended - T).to(torch.int32).to(device)
    return Fp8Case(q, k_codes, k_exp, v_codes, v_exp, lengths0, k_new, v_new, float(D) ** -0.5)


def paged_layout(B: int, T_cap: int, page_size: int, seed: int, spare_pages: Optional[int] = None):
    """Seeded block table for B sequences of capacity T_cap in pages of
    page_size tokens: block j of sequence b gets a distinct page drawn by a
    permutation, and ``spare_pages`` more pages (default: one sequence's
    worth) are never listed.  Returns (block_table [B, T_cap / P] int32 on
    the CPU, num_pages)."""
    P = int(page_size)
    assert T_cap % P == 0, "capacity must be a whole number of pages"
    nb = T_cap // P
    spare = nb if spare_pages is None else int(spare_pages)
    num_pages = B * nb + spare
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    table = torch.randperm(num_pages, generator=gen)[:B * nb].view(B, nb).to(torch.int32)
    return table, num_pages


def to_pages(x: torch.Tensor, table: torch.Tensor, page_size: int, num_pages: int) -> torch.Tensor:
    """Scatter per-token rows x [B, Hkv, T_cap, ...] into a pool
    [num_pages, Hkv, P, ...] under ``table``.  Pages no sequence lists hold
    a poison value: NaN for floats, the E4M3 NaN code 0x7F for uint8 codes,
    127 for int8 exponents."""
    B, Hkv, T_cap = x.shape[:3]
    rest = tuple(x.shape[3:])
    P = int(page_size)
    nb = T_cap // P
    fill = float("nan") if x.dtype.is_floating_point else (0x7F if x.dtype == torch.uint8 else 127)
    pool = torch.full((num_pages, Hkv, P) + rest, fill, dtype=x.dtype, device=x.device)
    blocks = x.reshape((B, Hkv, nb, P) + rest).transpose(1, 2)  # [B, nb, Hkv, P, ...]
    pool[table.view(-1).long().to(x.device)] = blocks.reshape((B * nb, Hkv, P) + rest)
    return pool


def make_paged(k_cache: torch.Tensor, v_cache: torch.Tensor, page_size: int, seed: int,
               spare_pages: Optional[int] = None):
    """Lay contiguous caches [B, Hkv, T_cap, D] out as a page pool
    (``paged_layout`` + ``to_pages``).  Returns (k_pages, v_pages,
    block_table) with pools [num_pages, Hkv, P, D] on the caches' device and
    block_table [B, T_cap / P] int32 on the CPU."""
    B, Hkv, T_cap, D = k_cache.shape
    table, num_pages = paged_layout(B, T_cap, page_size, seed, spare_pages)
    return (to_pages(k_cache, table, page_size, num_pages), to_pages(v_cache, table, page_size, num_pages),
            table)


def bf16_bits(t: torch.Tensor):
    """Raw bf16 bit patterns of a tensor as a numpy uint16 array (host)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def host_array(t: torch.Tensor):
    """Host numpy view in the encoding the oracle takes (float32 or bf16 bits)."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.detach().cpu().contiguous().numpy()
