"""Shared helpers of the GPU tests: run one decode step through the C ABI and
the same step through the oracle, on identical bytes."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
import multiquery_decode_attention_amd as kvd
from multiquery_decode_attention_amd import inputs


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def oracle_dtype(t: torch.Tensor) -> int:
    return oracle.BF16 if t.dtype == torch.bfloat16 else oracle.F32


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def gpu_step(case: inputs.Case, Hq: int, *, variant=None, splits=None, append=True,
             lengths=None, k_cache=None, v_cache=None, fused=False, reserve=False, unified_max=None):
    """Append (optional) then attend on the GPU, on fresh device copies of
    the case's tensors (the case itself is never modified).  Returns (out,
    k_cache, v_cache, lengths, status, plan)."""
    dev = torch.device("cuda")
    kc = (k_cache if k_cache is not None else case.k_cache).to(dev, copy=True).contiguous()
    vc = (v_cache if v_cache is not None else case.v_cache).to(dev, copy=True).contiguous()
    L = (lengths if lengths is not None else case.lengths0).to(dev, torch.int32, copy=True).contiguous()
    cache = kvd.KVCache(kc, vc, L, Hq)
    try:
        if variant is not None:
            cache.set_variant(variant)
        if splits is not None:
            cache.set_num_splits(splits)
        if unified_max is not None:
            cache.set_unified_max(unified_max)
        if reserve:  # twice: binding and allocation happen once
            cache.reserve()
            cache.reserve()
        plan = cache.plan()
        kn, vn = case.k_new.to(dev).contiguous(), case.v_new.to(dev).contiguous()
        if append and fused:
            out = cache.step(kn, vn, case.q.to(dev).contiguous(), scale=case.scale)
        else:
            if append:
                cache.append(kn, vn)
            out = cache.attend(case.q.to(dev).contiguous(), scale=case.scale)
        status = cache.status()
        torch.cuda.synchronize()
    finally:
        cache.close()
    return out, kc, vc, L, status, plan


def oracle_step(case: inputs.Case, *, append=True, lengths=None, rows=None):
    """The same step on the CPU oracle: numpy append, then fp64 attention.
    Returns (out_f64, k_after, v_after, lengths_after) as host arrays."""
    t0 = time.time()
    k = inputs.host_array(case.k_cache)
    v = inputs.host_array(case.v_cache)
    L = (lengths if lengths is not None else case.lengths0).cpu().numpy().astype(np.int32)
    if append:
        k, v, L, _ = oracle.append(k, v, L, inputs.host_array(case.k_new), inputs.host_array(case.v_new))
    out = oracle.decode_attention(inputs.host_array(case.q), k, v, L, case.scale,
                                  oracle_dtype(case.q), rows=rows)
    say(f"oracle done in {time.time() - t0:.1f}s")
    return out, k, v, L
