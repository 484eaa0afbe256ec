"""The allocation-free step (kvdecode_append_attend_noalloc) against the
allocating one (kvdecode_append_attend), through the C ABI.

Both run the same kernels on the same plan, so the outputs, caches and
lengths must agree bit for bit; the output is also checked against the fp64
oracle to its dtype's tolerance.  Two calls in a row on one GPU, the second
with a smaller input, so the second meets the static buffer as the first
left it.  The buffer's error word is reported by kvdecode_status and
cleared by it.
"""
import ctypes

import numpy as np
import pytest
import torch

import multiquery_decode_attention_amd as kvd
import oracle
from multiquery_decode_attention_amd import inputs
from conftest import rel_err_rows
from gpu_helpers import say, to_f64

pytestmark = pytest.mark.gpu


def one_step(case, Hq, noalloc, lengths=None, splits=0):
    """One decode step on fresh device copies of the case, through the C
    ABI (splits > 0: that split count forced).  Returns (out, k_cache,
    v_cache, lengths, status)."""
    lib = kvd.library()
    dev = torch.device("cuda")
    kc, vc = case.k_cache.to(dev, copy=True), case.v_cache.to(dev, copy=True)
    L = (case.lengths0 if lengths is None else lengths).to(dev, torch.int32, copy=True)
    kn, vn, q = (t.to(dev).contiguous() for t in (case.k_new, case.v_new, case.q))
    out = torch.empty_like(q)
    B, Hkv, T_cap, D = kc.shape
    desc = kvd.kvdecode_desc_t(B, Hq, Hkv, D, T_cap, kvd.KVD_BF16 if kc.dtype == torch.bfloat16 else kvd.KVD_F32,
                               kc.data_ptr(), vc.data_ptr(), L.data_ptr())
    h = ctypes.c_void_p()
    assert lib.kvdecode_create(ctypes.byref(desc), ctypes.byref(h)) == kvd.KVD_OK
    if splits:
        assert lib.kvdecode_set_num_splits(h, splits) == kvd.KVD_OK
    stream = torch.cuda.current_stream().cuda_stream
    fn = lib.kvdecode_append_attend_noalloc if noalloc else lib.kvdecode_append_attend
    rc = fn(h, kn.data_ptr(), vn.data_ptr(), q.data_ptr(), out.data_ptr(), ctypes.c_float(case.scale), stream)
    assert rc == kvd.KVD_OK, kvd.kvdecode_strerror(rc)
    status = lib.kvdecode_status(h, stream)
    torch.cuda.synchronize()
    assert lib.kvdecode_destroy(h) == kvd.KVD_OK
    return out, kc, vc, L, status


def check_against_allocating_step(case, Hq, tol, name, splits=0):
    say(f"noalloc {name}: B={case.q.shape[0]} Hq={Hq} Hkv={case.k_cache.shape[1]} D={case.q.shape[2]} "
        f"T_cap={case.k_cache.shape[2]} {case.q.dtype} splits={splits}")
    got = one_step(case, Hq, noalloc=True, splits=splits)
    want = one_step(case, Hq, noalloc=False, splits=splits)
    assert got[4] == kvd.KVD_OK and want[4] == kvd.KVD_OK, (got[4], want[4])
    for a, b, what in zip(got[:4], want[:4], ("output", "K cache", "V cache", "lengths")):
        assert torch.equal(a, b), f"{name}: {what} differs from kvdecode_append_attend's"
    k2, v2, L2, _ = oracle.append(inputs.host_array(case.k_cache), inputs.host_array(case.v_cache),
                                  case.lengths0.numpy(), inputs.host_array(case.k_new), inputs.host_array(case.v_new))
    dt = oracle.BF16 if case.q.dtype == torch.bfloat16 else oracle.F32
    ref = oracle.decode_attention(inputs.host_array(case.q), k2, v2, L2, case.scale, dt)
    err = rel_err_rows(to_f64(got[0]), ref)
    say(f"noalloc {name}: bitwise equal to the allocating step, row-relative error {err:.2e} (tol {tol:.0e})")
    assert err <= tol, err


def test_noalloc_matches_allocating_step_twice_second_smaller():
    """A long-context multiquery step (48 heads, d = 256, many splits), then
    a smaller grouped-query one (d = 128, ragged lengths), then the fp32
    tiny workload: each bitwise equal to kvdecode_append_attend."""
    big = inputs.make_case(4, 48, 1, 256, 16384, [16384, 9000, 16000, 3], "bf16", seed=501)
    small = inputs.make_case(3, 16, 4, 128, 512, [512, 100, 31], "bf16", seed=502, k_scale=3.0)
    check_against_allocating_step(big, 48, 2e-2, "long-context MQA")
    check_against_allocating_step(small, 16, 2e-2, "smaller GQA")
    tiny = inputs.make_workload_case(inputs.WORKLOADS["tiny_mqa_f32"], device="cpu")
    check_against_allocating_step(tiny, 8, 1e-3, "tiny fp32")


def test_noalloc_single_split_steps():
    """One-split steps (no combine; the last workgroup of each sequence
    advances its length on a per-sequence counter in the static buffer),
    three in a row on the LDS and VALU kernels: each bitwise equal to
    kvdecode_append_attend, so every step found the counters at zero."""
    small = inputs.make_case(3, 16, 4, 128, 512, [512, 100, 31], "bf16", seed=504, k_scale=3.0)
    tiny = inputs.make_workload_case(inputs.WORKLOADS["tiny_mqa_f32"], device="cpu")
    for rep in range(3):
        check_against_allocating_step(small, 16, 2e-2, f"smaller GQA one split #{rep}", splits=1)
        check_against_allocating_step(tiny, 8, 1e-3, f"tiny fp32 one split #{rep}", splits=1)


def test_noalloc_errors_are_sticky_until_status():
    """A step that finds a sequence at capacity sets the buffer's error word:
    kvdecode_status reports KVD_ECAPACITY and clears it, and the next clean
    step reports KVD_OK."""
    case = inputs.make_case(2, 8, 1, 128, 64, [64, 10], "bf16", seed=503)
    full = torch.tensor([64, 9], dtype=torch.int32)
    out, kc, vc, L, status = one_step(case, 8, noalloc=True, lengths=full)
    assert status == kvd.KVD_ECAPACITY
    assert L.cpu().tolist() == [64, 10]
    out, kc, vc, L, status = one_step(case, 8, noalloc=True)
    assert status == kvd.KVD_OK
