"""GPU parity of the several-new-tokens step (kvdecode_append_attend_multi).

T_q drafted tokens per sequence are appended and their T_q queries attend
causally (query i over the cache and new tokens 0..i).  Compared with the
oracle's append_multi (bit for bit) and decode_attention_multi (to the
bf16 / fp32 tolerance), on both partial kernels, contiguous and paged,
with lengths and split counts that leave some splits without any token for
the earlier queries.
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


def multi_step(case, Hq, *, variant="auto", splits=None, page_size=0, reserve=0):
    dev = torch.device("cuda")
    L = case.lengths0.to(dev, torch.int32, copy=True)
    if page_size:
        kc, vc, bt = inputs.make_paged(case.k_cache, case.v_cache, page_size, seed=3)
        kc, vc, btd = kc.to(dev, copy=True), vc.to(dev, copy=True), bt.to(dev)
        cache = kvd.KVCache(kc, vc, L, Hq, block_table=btd)
    else:
        kc, vc, bt = case.k_cache.to(dev, copy=True), case.v_cache.to(dev, copy=True), None
        cache = kvd.KVCache(kc, vc, L, Hq)
    try:
        cache.set_variant(VARIANTS[variant])
        if splits is not None:
            cache.set_num_splits(splits)
        if reserve:
            cache.reserve(reserve)
        kn, vn, q = (t.to(dev).contiguous() for t in (case.k_new, case.v_new, case.q))
        out = cache.step_multi(kn, vn, q, scale=case.scale)
        status = cache.status()
        torch.cuda.synchronize()
    finally:
        cache.close()
    if page_size:  # back to the contiguous caches the pools stand for
        kc = torch.as_tensor(oracle.gather_pages(inputs.host_array(kc), bt.numpy()))
        vc = torch.as_tensor(oracle.gather_pages(inputs.host_array(vc), bt.numpy()))
    else:
        kc, vc = torch.as_tensor(inputs.host_array(kc)), torch.as_tensor(inputs.host_array(vc))
    return out, kc.numpy(), vc.numpy(), L.cpu().numpy(), status


def oracle_multi(case):
    k, v = inputs.host_array(case.k_cache), inputs.host_array(case.v_cache)
    L0 = case.lengths0.cpu().numpy()
    k2, v2, L2, a = oracle.append_multi(k, v, L0, inputs.host_array(case.k_new), inputs.host_array(case.v_new))
    dt = oracle.BF16 if case.q.dtype == torch.bfloat16 else oracle.F32
    ref = oracle.decode_attention_multi(inputs.host_array(case.q), k2, v2, L2, a, case.scale, dt)
    return ref, k2, v2, L2, a


def check_multi(case, Hq, name, expect_status=kvd.KVD_OK, **kw):
    B, _, T_q, D = case.q.shape
    say(f"{name}: B={B} Hq={Hq} T_q={T_q} T_cap={case.k_cache.shape[2]} D={D} {kw}")
    out, kc, vc, L, status = multi_step(case, Hq, **kw)
    ref, k2, v2, L2, a = oracle_multi(case)
    assert status == expect_status
    assert np.array_equal(L, L2)
    assert np.array_equal(kc, k2) and np.array_equal(vc, v2), "caches differ after the append"
    tol = TOL_BF16 if case.q.dtype == torch.bfloat16 else TOL_F32
    err = rel_err_rows(to_f64(out), ref)
    say(f"{name}: max row-relative error {err:.3e} (tol {tol:.0e})")
    assert err <= tol, err
    return out


@pytest.mark.parametrize("name,T_q,sample", [("palm_mqa_bf16", 4, None), ("longctx_mqa_bf16", 4, None),
                                           ("llama13b_mha_bf16", 8, 8), ("ragged_gqa_bf16", 4, 16)])
def test_multi_token_full_size(name, T_q, sample):
    """The workloads at full size with T_q new tokens per sequence (the
    step `bench.py --new-tokens T_q` times, automatic plan): the append bit
    for bit on the whole cache, attention against the oracle on every
    sequence or on a seeded sample of them."""
    w = inputs.WORKLOADS[name]
    L0 = inputs.attended_lengths(w) - T_q
    say(f"multi full {name}: B={w.B} Hq={w.Hq} T_q={T_q} T_cap={w.T_cap}")
    case = inputs.make_multi_case(w.B, w.Hq, w.Hkv, w.D, w.T_cap, L0, T_q, w.dtype, seed=w.seed, device="cuda")
    out, kc, vc, L, status = multi_step(case, w.Hq)
    assert status == kvd.KVD_OK
    k2, v2, L2, a = oracle.append_multi(inputs.host_array(case.k_cache), inputs.host_array(case.v_cache),
                                        L0.numpy(), inputs.host_array(case.k_new), inputs.host_array(case.v_new))
    assert np.array_equal(L, L2)
    assert np.array_equal(kc, k2) and np.array_equal(vc, v2), "caches differ after the append"
    sel = np.arange(w.B) if sample is None else np.sort(np.random.default_rng(w.seed).choice(w.B, sample, replace=False))
    ref = oracle.decode_attention_multi(inputs.host_array(case.q)[sel], k2[sel], v2[sel], L2[sel], a[sel], case.scale,
                                        oracle.BF16)
    err = rel_err_rows(to_f64(out)[sel], ref)
    say(f"multi full {name}: {len(sel)} sequences checked, max row-relative error {err:.3e}")
    assert err <= TOL_BF16, err


@pytest.mark.parametrize("T_q", [2, 4, 8, 16])
@pytest.mark.parametrize("shape", ["palm_like", "gqa", "mha"])
def test_multi_token_shapes(shape, T_q):
    B, Hq, Hkv, D, T_cap, L0 = {
        "palm_like": (3, 48, 1, 256, 2048, [2000, 31, 700]),
        "gqa": (4, 64, 8, 128, 1024, [1000, 0, 33, 513]),
        "mha": (2, 40, 40, 128, 512, [400, 95]),
    }[shape]
    case = inputs.make_multi_case(B, Hq, Hkv, D, T_cap, L0, T_q, "bf16", seed=T_q * 7 + len(shape))
    check_multi(case, Hq, f"multi {shape} T_q={T_q}")


@pytest.mark.parametrize("variant", ["lds", "valu"])
@pytest.mark.parametrize("splits", [1, 3, 9])
def test_multi_token_empty_splits(variant, splits):
    """Lengths just below tile edges: the early queries' last tokens end in
    tiles (and splits) that the later queries reach past."""
    L0 = [31, 60, 95, 1, 64]
    case = inputs.make_multi_case(len(L0), 16, 2, 128, 256, L0, 6, "bf16", seed=40 + splits)
    check_multi(case, 16, f"multi edges {variant} S={splits}", variant=variant, splits=splits)


@pytest.mark.parametrize("splits", [20, 40])
def test_multi_token_many_splits_d256(splits):
    """d = 256 with more than 16 splits (several split groups per row in the
    combine): early queries whose last tokens end before later splits
    (empty splits, log-sum-exp -inf) must weigh those splits 0."""
    L0 = [31, 700, 95, 1, 1200]
    case = inputs.make_multi_case(len(L0), 48, 1, 256, 1280, L0, 4, "bf16", seed=60 + splits)
    check_multi(case, 48, f"multi d256 S={splits}", variant="lds", splits=splits)


def test_multi_token_fp32_and_paged():
    case = inputs.make_multi_case(2, 8, 1, 64, 256, [100, 3], 5, "f32", seed=61)
    check_multi(case, 8, "multi fp32 valu")
    case = inputs.make_multi_case(3, 48, 1, 256, 512, [200, 33, 480], 4, "bf16", seed=62)
    check_multi(case, 48, "multi paged", page_size=64)


@pytest.mark.parametrize("T_q,reserve", [(4, 4), (4, 16), (16, 16)])
def test_multi_token_after_reserve(T_q, reserve):
    """kvdecode_reserve for steps of up to `reserve` new tokens, then a step
    of T_q: same results as without the reservation."""
    case = inputs.make_multi_case(3, 48, 1, 256, 1024, [1000, 31, 500], T_q, "bf16", seed=70 + T_q)
    check_multi(case, 48, f"multi reserve {reserve} T_q={T_q}", reserve=reserve)


def test_multi_token_without_room():
    case = inputs.make_multi_case(3, 16, 2, 128, 128, [126, 124, 10], 4, "bf16", seed=63)
    check_multi(case, 16, "multi overflow", expect_status=kvd.KVD_ECAPACITY)


def test_one_new_token_matches_the_one_token_step_bitwise():
    w = inputs.WORKLOADS["ragged_gqa_bf16"]
    single = inputs.make_workload_case(w, device="cpu", B=6)
    multi = inputs.MultiCase(single.q[:, :, None].contiguous(), single.k_cache, single.v_cache, single.lengths0,
                             single.k_new[:, :, None].contiguous(), single.v_new[:, :, None].contiguous(),
                             single.scale)
    out_1, kc1, vc1, L1, st1, _ = gpu_step(single, w.Hq, fused=True)
    out_m, kcm, vcm, Lm, stm = multi_step(multi, w.Hq)
    assert st1 == stm == kvd.KVD_OK
    assert torch.equal(out_1.cpu().view(torch.int16), out_m[:, :, 0].cpu().contiguous().view(torch.int16))
    assert np.array_equal(inputs.host_array(kc1), kcm) and np.array_equal(L1.cpu().numpy(), Lm)
