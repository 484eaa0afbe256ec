"""GPU parity of the exchange kernel on bf16 caches (KVD_VARIANT_XCHG).

The four waves of a workgroup split each 64-token tile by tokens for the
scores and by value columns for the weighted sum, trading weights through
LDS.  Forced through kvdecode_set_variant on query groups of 1-4 16-row
blocks and several row groups, lengths on and next to the kernel's 16-token
block and 64-token tile edges, forced split counts, the fused step, several
new tokens per sequence, paged caches and the out-of-range length; every
output compared with the fp64 oracle to the bf16 tolerance and every append
bit for bit.
"""
import numpy as np
import pytest
import torch

import multiquery_decode_attention_amd as kvd
from multiquery_decode_attention_amd import inputs
from conftest import TOL_BF16, rel_err_rows
from gpu_helpers import gpu_step, oracle_step, say, to_f64
from test_gpu_multi import check_multi
from test_gpu_paged import check_paged
from test_gpu_parity import check_case

pytestmark = pytest.mark.gpu

XCHG = kvd.KVD_VARIANT_XCHG


@pytest.mark.parametrize("Hq,Hkv,D", [(48, 1, 256), (32, 1, 256), (16, 2, 256), (96, 1, 256), (64, 1, 128),
                                     (80, 1, 128), (40, 2, 128), (17, 1, 256)])
@pytest.mark.parametrize("splits", [None, 1, 3])
def test_xchg_bf16_row_groups_and_edges(Hq, Hkv, D, splits):
    """One to four row blocks per workgroup, two row groups (96 rows at
    d = 256, 80 at d = 128), a padded group (17 rows); lengths attended (the
    new token included) land the fused append in slots 0, 16 and 64."""
    lengths = [1, 15, 16, 17, 48, 63, 64, 65, 100, 129, 250]
    case = inputs.make_case(len(lengths), Hq, Hkv, D, 256, lengths, "bf16", seed=170 + Hq + D)
    for fused in (True, False):
        _, _, plan = check_case(case, Hq, f"bf16 xchg Hq={Hq} Hkv={Hkv} D={D} S={splits} fused={fused}",
                                variant=XCHG, splits=splits, fused=fused)
        assert plan["variant"] == "xchg"


@pytest.mark.parametrize("name,B", [("palm_mqa_bf16", 3), ("ragged_gqa_bf16", 4), ("llama13b_mha_bf16", 1),
                                    ("longctx_mqa_bf16", 1)])
def test_xchg_bf16_workloads(name, B):
    w = inputs.WORKLOADS[name]
    case = inputs.make_workload_case(w, device="cpu", B=B)
    if name == "longctx_mqa_bf16":  # keep the CPU copy small: 8192 tokens
        case = inputs.make_case(1, w.Hq, w.Hkv, w.D, 8192, [8192], "bf16", seed=w.seed)
    check_case(case, w.Hq, f"{name}/xchg", variant=XCHG, fused=True)


@pytest.mark.parametrize("phi", [0.0, -40.0, 1e4])
def test_xchg_bf16_unified_max(phi):
    case = inputs.make_case(3, 48, 1, 256, 2048, [2048, 1000, 33], "bf16", seed=171)
    check_case(case, 48, f"bf16 xchg unified max {phi}", variant=XCHG, unified_max=phi)


def test_xchg_bf16_fused_step_with_out_of_range_length():
    """A length past capacity with the append fused into the exchange
    kernel: no append for that sequence, attention clamped to capacity,
    KVD_ELENGTH; the other sequence steps normally."""
    case = inputs.make_case(2, 48, 1, 256, 96, [96, 41], "bf16", seed=172)
    L_bad = torch.tensor([1000, 40], dtype=torch.int32)
    out, kc, vc, L, status, plan = gpu_step(case, 48, lengths=L_bad, fused=True, variant=XCHG)
    assert plan["variant"] == "xchg"
    assert status == kvd.KVD_ELENGTH
    assert L.cpu().tolist() == [1000, 41]
    ref, k2, v2, _ = oracle_step(case, lengths=torch.tensor([96, 40], dtype=torch.int32))
    assert np.array_equal(inputs.host_array(kc), k2) and np.array_equal(inputs.host_array(vc), v2)
    assert rel_err_rows(to_f64(out), ref) <= TOL_BF16


@pytest.mark.parametrize("T_q", [2, 4, 8, 16])
@pytest.mark.parametrize("shape", ["palm_like", "gqa"])
def test_xchg_bf16_multi_token(shape, T_q):
    """Several new tokens per sequence: T_q times the query rows of a group,
    so 16 new tokens at 48 heads take several row groups."""
    B, Hq, Hkv, D, T_cap, L0 = {
        "palm_like": (3, 48, 1, 256, 2048, [2000, 31, 700]),
        "gqa": (4, 64, 8, 128, 1024, [1000, 0, 33, 513]),
    }[shape]
    case = inputs.make_multi_case(B, Hq, Hkv, D, T_cap, L0, T_q, "bf16", seed=T_q * 11 + len(shape))
    check_multi(case, Hq, f"bf16 xchg multi {shape} T_q={T_q}", variant="xchg")


@pytest.mark.parametrize("splits", [1, 3, 9])
def test_xchg_bf16_multi_token_empty_splits(splits):
    L0 = [31, 60, 95, 1, 64]
    case = inputs.make_multi_case(len(L0), 16, 2, 128, 256, L0, 6, "bf16", seed=140 + splits)
    check_multi(case, 16, f"bf16 xchg multi edges S={splits}", variant="xchg", splits=splits)


@pytest.mark.parametrize("page", [32, 64, 256])
@pytest.mark.parametrize("fused", [True, False])
def test_xchg_bf16_paged(page, fused):
    """Pages of 32 tokens cut the 64-token tiles in two;
    the pages of a sequence are shuffled in the pool."""
    case = inputs.make_case(3, 48, 1, 256, 1024, [1024, 500, 17], "bf16", seed=173 + page)
    _, plan = check_paged(case, 48, page, f"bf16 xchg paged {page}", variant="xchg", fused=fused)
    assert plan["variant"] == "xchg"


def test_xchg_bf16_multi_token_paged():
    case = inputs.make_multi_case(3, 48, 1, 256, 512, [200, 33, 480], 4, "bf16", seed=174)
    check_multi(case, 48, "bf16 xchg multi paged", variant="xchg", page_size=32)


def test_xchg_bf16_multi_token_full_size():
    """The long-context workload with 4 new tokens per sequence through the
    exchange kernel, every sequence checked."""
    w = inputs.WORKLOADS["longctx_mqa_bf16"]
    T_q = 4
    L0 = inputs.attended_lengths(w) - T_q
    say(f"bf16 xchg multi full: B={w.B} Hq={w.Hq} T_q={T_q} T_cap={w.T_cap}")
    case = inputs.make_multi_case(w.B, w.Hq, w.Hkv, w.D, w.T_cap, L0, T_q, w.dtype, seed=w.seed, device="cuda")
    check_multi(case, w.Hq, "bf16 xchg multi longctx", variant="xchg")
