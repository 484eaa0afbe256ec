"""GPU parity of the paged KV cache, through the C ABI, against the oracle.

The caches are laid out as page pools with a seeded random block table
(inputs.make_paged); the oracle attends over the gathered pools and appends
through the block table (oracle.gather_pages / append_paged, pinned on the
CPU).  Appends are checked bit for bit on the whole pool; attention to the
bf16/fp32 tolerances.  A paged step also has to reproduce the contiguous
step's output bit for bit: the plan and the arithmetic are the same, only
the addresses differ.
"""
import numpy as np
import pytest
import torch

import multiquery_decode_attention_amd as kvd
import oracle
from multiquery_decode_attention_amd import inputs
from conftest import TOL_BF16, TOL_F32, rel_err_rows
from gpu_helpers import gpu_step, say, to_f64

pytestmark = pytest.mark.gpu

VARIANTS = {"auto": kvd.KVD_VARIANT_AUTO, "valu": kvd.KVD_VARIANT_VALU, "lds": kvd.KVD_VARIANT_LDS}


def paged_step(case, Hq, page_size, *, seed=11, variant="auto", splits=None, fused=True,
               lengths=None, table_edit=None):
    """One step on fresh device copies of the case laid out in pages.
    Returns (out, k_pages, v_pages, block_table, lengths, status, plan,
    k_pages_before, v_pages_before)."""
    dev = torch.device("cuda")
    kp, vp, bt = inputs.make_paged(case.k_cache, case.v_cache, page_size, seed)
    if table_edit is not None:
        table_edit(bt)
    k0, v0 = inputs.host_array(kp), inputs.host_array(vp)
    kp, vp = kp.to(dev, copy=True), vp.to(dev, copy=True)
    btd = bt.to(dev, copy=True)
    L = (lengths if lengths is not None else case.lengths0).to(dev, torch.int32, copy=True)
    cache = kvd.KVCache(kp, vp, L, Hq, block_table=btd)
    try:
        cache.set_variant(VARIANTS[variant])
        if splits is not None:
            cache.set_num_splits(splits)
        plan = cache.plan()
        kn, vn, q = (t.to(dev).contiguous() for t in (case.k_new, case.v_new, case.q))
        if fused:
            out = cache.step(kn, vn, q, scale=case.scale)
        else:
            cache.append(kn, vn)
            out = cache.attend(q, scale=case.scale)
        status = cache.status()
        torch.cuda.synchronize()
    finally:
        cache.close()
    return out, kp, vp, bt, L, status, plan, k0, v0


def oracle_paged_step(case, k0, v0, bt, lengths=None):
    L = (lengths if lengths is not None else case.lengths0).cpu().numpy().astype(np.int32)
    k2, v2, L2, _ = oracle.append_paged(k0, v0, bt.numpy(), L, inputs.host_array(case.k_new),
                                        inputs.host_array(case.v_new))
    dt = oracle.BF16 if case.q.dtype == torch.bfloat16 else oracle.F32
    ref = oracle.decode_attention_paged(inputs.host_array(case.q), k2, v2, bt.numpy(), L2, case.scale, dt)
    return ref, k2, v2, L2


def same_bits(a, b):
    """Bitwise equality of two host arrays (the pools' spare pages hold NaN)."""
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and a.dtype == b.dtype and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def check_paged(case, Hq, page_size, name, **kw):
    say(f"{name}: paged B={case.q.shape[0]} Hq={Hq} T_cap={case.k_cache.shape[2]} page={page_size} {kw}")
    out, kp, vp, bt, L, status, plan, k0, v0 = paged_step(case, Hq, page_size, **kw)
    say(f"{name}: gpu done, plan={plan}, status={status}")
    ref, k2, v2, L2 = oracle_paged_step(case, k0, v0, bt, kw.get("lengths"))
    assert status == kvd.KVD_OK
    assert np.array_equal(L.cpu().numpy(), L2)
    assert same_bits(inputs.host_array(kp), k2), "K pool differs after append"
    assert same_bits(inputs.host_array(vp), v2), "V pool differs after append"
    tol = TOL_BF16 if case.q.dtype == torch.bfloat16 else TOL_F32
    err = rel_err_rows(to_f64(out), ref)
    say(f"{name}: max row-relative error {err:.3e} (tol {tol:.0e})")
    assert err <= tol, err
    return out, plan


@pytest.mark.parametrize("name,B,page", [("ragged_gqa_bf16", 8, 64), ("palm_mqa_bf16", 3, 256),
                                         ("llama13b_mha_bf16", 2, 128), ("tiny_mqa_f32", 1, 32)])
@pytest.mark.parametrize("fused", [True, False])
def test_paged_workloads(name, B, page, fused):
    w = inputs.WORKLOADS[name]
    case = inputs.make_workload_case(w, device="cpu", B=B)
    check_paged(case, w.Hq, page, f"{name}/paged{page}", fused=fused)


def test_paged_long_context_long_splits():
    """d = 256 with long splits: the two-workgroups-per-CU configuration,
    more than 64 tiles per split (the block-table register is reloaded)."""
    w = inputs.WORKLOADS["longctx_mqa_bf16"]
    case = inputs.make_case(1, w.Hq, w.Hkv, w.D, 16384, [16384], "bf16", seed=w.seed)
    check_paged(case, w.Hq, 1024, "longctx/paged1024/S2", splits=2)
    check_paged(case, w.Hq, 512, "longctx/paged512")


@pytest.mark.parametrize("fused", [True, False])
def test_paged_largest_pages(fused):
    """Pages of 65536 tokens, the largest size the header accepts (two
    blocks per sequence, shuffled; the second sequence ends inside its
    second page)."""
    case = inputs.make_case(2, 8, 1, 64, 2 * 65536, [2 * 65536, 70001], "bf16", seed=65536)
    check_paged(case, 8, 65536, "paged65536", fused=fused)


def test_paged_ragged_full_size():
    w = inputs.WORKLOADS["ragged_gqa_bf16"]
    case = inputs.make_workload_case(w, device="cpu")
    check_paged(case, w.Hq, 256, "ragged_gqa_bf16/full/paged256")


@pytest.mark.parametrize("variant", ["lds", "valu"])
@pytest.mark.parametrize("splits", [1, 5])
def test_paged_variants_and_splits(variant, splits):
    lengths = [1, 31, 32, 33, 64, 65, 127, 128, 200, 255]
    case = inputs.make_case(len(lengths), 16, 2, 128, 256, lengths, "bf16", seed=50 + splits)
    check_paged(case, 16, 32, f"paged32 {variant} S={splits}", variant=variant, splits=splits)


@pytest.mark.parametrize("name,B,page", [("ragged_gqa_bf16", 6, 64), ("palm_mqa_bf16", 2, 128),
                                         ("tiny_mqa_f32", 1, 32)])
def test_paged_equals_contiguous_bitwise(name, B, page):
    w = inputs.WORKLOADS[name]
    case = inputs.make_workload_case(w, device="cpu", B=B)
    out_c, *_ = gpu_step(case, w.Hq, fused=True)
    out_p, *_ = paged_step(case, w.Hq, page)
    assert torch.equal(out_c.cpu().view(torch.int16) if out_c.dtype == torch.bfloat16 else out_c.cpu(),
                       out_p.cpu().view(torch.int16) if out_p.dtype == torch.bfloat16 else out_p.cpu())


@pytest.mark.parametrize("variant", ["lds", "valu"])
def test_bad_block_table_entry_is_reported(variant):
    """An entry in use outside the pool is read as page 0 (memory-safe) and
    reported; sequences with valid tables are unaffected."""
    lengths = [100, 70]
    case = inputs.make_case(2, 8, 1, 128, 128, lengths, "bf16", seed=61)

    def corrupt(bt):
        bt[0, 1] = 10_000  # block 1 of sequence 0 (tokens 32..63) is in use

    out, kp, vp, bt, L, status, plan, k0, v0 = paged_step(case, 8, 32, variant=variant,
                                                         table_edit=corrupt)
    assert status == kvd.KVD_EPAGE
    ref, *_ = oracle_paged_step(case, k0, v0, bt)
    assert rel_err_rows(to_f64(out)[1:], ref[1:]) <= TOL_BF16
