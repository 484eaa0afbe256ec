"""The benchmark's byte accounting against the pages' worked numbers."""
import json
import math
import os

import pytest

from multiquery_decode_attention_amd import traffic
from multiquery_decode_attention_amd.inputs import WORKLOADS, attended_lengths

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                    "byte_model_worked_examples.json")
CASES = {c["id"]: c for c in json.load(open(GOLD))["cases"]}


def test_kv_bytes_per_token():
    c = CASES["kv_bytes_per_token_toy_model_int8"]
    got = traffic.kv_bytes_per_token(**c["args"])
    assert got == c["exact"]
    assert got == pytest.approx(c["printed"], rel=c["rel_tol"])


def test_kv_bytes_per_sequence():
    c = CASES["kv_bytes_per_sequence_128k"]
    a = dict(c["args"])
    n = a.pop("tokens")
    assert traffic.kv_bytes_per_token(**a) * n == pytest.approx(c["printed"], rel=c["rel_tol"])


def test_max_batch():
    c = CASES["max_batch_toy_model_int8_128k"]
    a = dict(c["args"])
    per_seq = traffic.kv_bytes_per_token(a["layers"], a["kv_heads"], a["head_dim"], a["elem_bytes"]) * a["tokens"]
    free = a["chips"] * a["hbm_per_chip"] - a["param_bytes"]
    assert math.floor(free / per_seq) == c["printed"]
    per_seq1 = traffic.kv_bytes_per_token(a["layers"], 1, a["head_dim"], a["elem_bytes"]) * a["tokens"]
    assert math.floor(free / per_seq1) == c["printed_one_kv_head"]


def test_step_bounds():
    c = CASES["step_lower_bound_batch4"]
    assert traffic.memory_bound_step_seconds(**c["args"]) == pytest.approx(c["printed"], rel=c["rel_tol"])
    c = CASES["step_estimate_batch256"]
    assert traffic.step_seconds_with_flops(**c["args"]) == pytest.approx(c["printed"], rel=c["rel_tol"])


def test_workload_byte_counts():
    """Attend bytes of the fixed-length workloads (closed form)."""
    w = WORKLOADS["longctx_mqa_bf16"]
    L = attended_lengths(w).tolist()
    assert traffic.attend_bytes(w.B, w.Hq, w.Hkv, w.D, 2, L) == 2 * 1 * 256 * 2 * 65536 * 8 + 2 * 8 * 48 * 256 * 2
    assert traffic.attend_bytes(w.B, w.Hq, w.Hkv, w.D, 2, L) == 537_264_128
    w = WORKLOADS["palm_mqa_bf16"]
    assert traffic.attend_bytes(w.B, w.Hq, w.Hkv, w.D, 2, attended_lengths(w).tolist()) == 137_363_456
    w = WORKLOADS["llama13b_mha_bf16"]
    assert traffic.attend_bytes(w.B, w.Hq, w.Hkv, w.D, 2, attended_lengths(w).tolist()) == 2_685_009_920
    w = WORKLOADS["tiny_mqa_f32"]
    assert traffic.attend_bytes(w.B, w.Hq, w.Hkv, w.D, 4, attended_lengths(w).tolist()) == 70_144
    # arithmetic intensity of the grouped step is about M FLOP per byte in bf16
    w = WORKLOADS["palm_mqa_bf16"]
    L = attended_lengths(w).tolist()
    ai = traffic.attend_flops(w.Hq, w.D, L) / traffic.attend_bytes(w.B, w.Hq, w.Hkv, w.D, 2, L)
    assert ai == pytest.approx(w.Hq // w.Hkv, rel=0.03)


def test_ragged_lengths_recipe():
    w = WORKLOADS["ragged_gqa_bf16"]
    L = attended_lengths(w)
    assert L.min() >= 64 and L.max() <= 8192 and len(set(L.tolist())) > 100
    assert attended_lengths(w).tolist() == L.tolist()  # seeded


def test_fp8_byte_counts():
    """fp8 cache: one byte per value plus an exponent byte per K and per V
    row; bf16 queries and outputs.  The long-context step reads a little
    over half the bf16 bytes."""
    w = WORKLOADS["longctx_mqa_bf16"]
    L = [65536] * 8
    kv = traffic.kv_read_bytes_fp8(w.Hkv, w.D, L)
    assert kv == 2 * 1 * (256 + 1) * 65536 * 8
    assert traffic.partial_pass_bytes_fp8(w.B, w.Hq, w.Hkv, w.D, L) == kv + 8 * 48 * 256 * 2
    assert traffic.attend_bytes_fp8(w.B, w.Hq, w.Hkv, w.D, L) == kv + 2 * 8 * 48 * 256 * 2
    ratio = kv / traffic.kv_read_bytes(w.Hkv, w.D, 2, L)
    assert ratio == pytest.approx(257 / 512)
    assert traffic.append_bytes_fp8(8, 1, 256) == 2 * 8 * 256 * 2 + 2 * 8 * 257
