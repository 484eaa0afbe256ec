"""Algorithmic byte and FLOP accounting of decode attention (used by the
benchmark's roofline figures).

The pages count attention traffic per head as: read Q, read the K and V
cache, write the output; the scores and probabilities never reach HBM when
the softmax is fused ("All About Transformer Inference", section on
attention cost, the Flash Attention fusion).  The KV cache of one token is
2 (keys and values) x layers x KV heads x head dim x bytes per element
(same page, section on memory, and its worked problem for the toy model).
"""
from __future__ import annotations

from typing import Sequence

MI355X_HBM_PEAK_GBPS = 8000.0      # HBM3E, 8 TB/s (published peak)
MI355X_BF16_DENSE_TFLOPS = 2500.0  # dense bf16 matrix peak


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: float) -> float:
    """Cache bytes of one token: keys and values of every layer and KV head."""
    return 2 * layers * kv_heads * head_dim * elem_bytes


def kv_read_bytes(kv_heads: int, head_dim: int, elem_bytes: int, lengths: Sequence[int]) -> int:
    """K and V bytes of every valid cached token of one layer's decode step."""
    return int(kv_bytes_per_token(1, kv_heads, head_dim, elem_bytes) * sum(int(n) for n in lengths))


def attend_bytes(B: int, Hq: int, Hkv: int, D: int, elem: int, lengths: Sequence[int]) -> int:
    """Whole attend pass: read K/V of the valid prefixes, read q, write out."""
    return kv_read_bytes(Hkv, D, elem, lengths) + 2 * B * Hq * D * elem


def partial_pass_bytes(B: int, Hq: int, Hkv: int, D: int, elem: int, lengths: Sequence[int]) -> int:
    """The split-KV partial kernel's algorithmic reads: K/V of the valid
    prefixes plus the queries (its partial outputs are implementation
    overhead, not counted)."""
    return kv_read_bytes(Hkv, D, elem, lengths) + B * Hq * D * elem


def append_bytes(B: int, Hkv: int, D: int, elem: int) -> int:
    """Read the new token's K and V, write them into the cache."""
    return 4 * B * Hkv * D * elem


# fp8 cache: one byte per value plus one exponent byte per K row and per V
# row; queries, outputs and the appended rows stay bf16.

def kv_read_bytes_fp8(kv_heads: int, head_dim: int, lengths: Sequence[int]) -> int:
    """K and V codes and exponents of every valid cached token."""
    return 2 * kv_heads * (head_dim + 1) * sum(int(n) for n in lengths)


def partial_pass_bytes_fp8(B: int, Hq: int, Hkv: int, D: int, lengths: Sequence[int]) -> int:
    """Partial-kernel reads over an fp8 cache: codes and exponents of the
    valid prefixes plus the bf16 queries."""
    return kv_read_bytes_fp8(Hkv, D, lengths) + B * Hq * D * 2


def attend_bytes_fp8(B: int, Hq: int, Hkv: int, D: int, lengths: Sequence[int]) -> int:
    """Whole attend pass over an fp8 cache (bf16 q in, bf16 out)."""
    return kv_read_bytes_fp8(Hkv, D, lengths) + 2 * B * Hq * D * 2


def append_bytes_fp8(B: int, Hkv: int, D: int) -> int:
    """Read the new bf16 K and V rows, write their codes and exponents."""
    return 2 * B * Hkv * D * 2 + 2 * B * Hkv * (D + 1)


def attend_flops(Hq: int, D: int, lengths: Sequence[int]) -> int:
    """2*D for the score and 2*D for the value product per (head, token)."""
    return 4 * Hq * D * sum(int(n) for n in lengths)


def memory_bound_step_seconds(batch: int, kv_bytes_per_seq: float, param_bytes: float,
                              chips: int, hbm_bytes_per_s: float) -> float:
    """Lower bound on a small-batch generate step: every parameter and every
    sequence's KV cache is loaded once (same page, section on latency and
    throughput estimates)."""
    return (batch * kv_bytes_per_seq + param_bytes) / (chips * hbm_bytes_per_s)


def step_seconds_with_flops(batch: int, kv_bytes_per_seq: float, param_count: float,
                            chips: int, hbm_bytes_per_s: float, flops_per_s: float) -> float:
    """Large-batch form: attention stays bandwidth bound, the MLP becomes
    compute bound at 2 FLOPs per parameter per token."""
    return (batch * kv_bytes_per_seq) / (chips * hbm_bytes_per_s) + \
        (2 * batch * param_count) / (chips * flops_per_s)
