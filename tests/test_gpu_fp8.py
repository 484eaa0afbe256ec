"""GPU parity of the fp8 (E4M3 + per-row power-of-two exponent) KV cache.

The cache is drawn as codes and exponents; the step's new bf16 rows are
quantized by the library's append and by the oracle's append_fp8, which
must agree bit for bit on every code, exponent and length.  Attention is
compared with the oracle's fp64 attention over the dequantized cache, to
the bf16 tolerance (the kernel widens codes to bf16 exactly; its error is
the bf16 rounding of the weights and of the output, as in the bf16 path).
"""
import numpy as np
import pytest
import torch

import multiquery_decode_attention_amd as kvd
import oracle
from multiquery_decode_attention_amd import inputs
from conftest import TOL_BF16, rel_err_rows
from gpu_helpers import say, to_f64

pytestmark = pytest.mark.gpu

# wave: each wave streams its own tiles for all query heads of its group
# (d >= 128; several row groups share tiles through L2); lds: the four waves
# share every tile; xchg: the waves split each 64-token tile by tokens for
# the scores and by columns for the values, exchanging weights in LDS
# (d >= 128)
VARIANTS = {"auto": kvd.KVD_VARIANT_AUTO, "wave": kvd.KVD_VARIANT_WAVE, "lds": kvd.KVD_VARIANT_LDS,
            "xchg": kvd.KVD_VARIANT_XCHG}


def fp8_step(case, Hq, *, fused=True, splits=None, lengths=None, unified_max=None, variant="auto"):
    dev = torch.device("cuda")
    kc, vc = case.k_codes.to(dev, copy=True), case.v_codes.to(dev, copy=True)
    ke, ve = case.k_exp.to(dev, copy=True), case.v_exp.to(dev, copy=True)
    L = (lengths if lengths is not None else case.lengths0).to(dev, torch.int32, copy=True)
    cache = kvd.KVCache(kc, vc, L, Hq, k_exp=ke, v_exp=ve)
    try:
        cache.set_variant(VARIANTS[variant])
        if splits is not None:
            cache.set_num_splits(splits)
        if unified_max is not None:
            cache.set_unified_max(unified_max)
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
    return out, kc, ke, vc, ve, L, status, plan


def oracle_fp8_step(case, lengths=None):
    L = (lengths if lengths is not None else case.lengths0).cpu().numpy().astype(np.int32)
    f32 = lambda t: t.float().cpu().numpy()
    kc, ke, vc, ve, L2, _ = oracle.append_fp8(case.k_codes.numpy(), case.k_exp.numpy(), case.v_codes.numpy(),
                                              case.v_exp.numpy(), L, f32(case.k_new), f32(case.v_new))
    ref = oracle.decode_attention_fp8(f32(case.q), kc, ke, vc, ve, L2, case.scale)
    return ref, kc, ke, vc, ve, L2


def check_fp8(case, Hq, name, **kw):
    say(f"{name}: fp8 B={case.q.shape[0]} Hq={Hq} Hkv={case.k_codes.shape[1]} "
        f"T_cap={case.k_codes.shape[2]} D={case.q.shape[2]} {kw}")
    out, kc, ke, vc, ve, L, status, plan = fp8_step(case, Hq, **kw)
    say(f"{name}: gpu done, plan={plan}, status={status}")
    ref, kc2, ke2, vc2, ve2, L2 = oracle_fp8_step(case, kw.get("lengths"))
    assert status == kvd.KVD_OK
    assert np.array_equal(L.cpu().numpy(), L2)
    assert np.array_equal(ke.cpu().numpy(), ke2) and np.array_equal(ve.cpu().numpy(), ve2), "exponents differ"
    assert np.array_equal(kc.cpu().numpy(), kc2), "K codes differ after append"
    assert np.array_equal(vc.cpu().numpy(), vc2), "V codes differ after append"
    err = rel_err_rows(to_f64(out), ref)
    say(f"{name}: max row-relative error {err:.3e} (tol {TOL_BF16:.0e})")
    assert err <= TOL_BF16, err
    return out, plan


# Workloads at full size with an fp8 cache: sequences whose attention the
# oracle checks (None: all; else a seeded sample of that many).
FP8_FULL = {"palm_mqa_bf16": None, "llama13b_mha_bf16": 8, "ragged_gqa_bf16": 16, "longctx_mqa_bf16": None}


@pytest.mark.parametrize("name", list(FP8_FULL))
def test_fp8_workload_full_size(name):
    """Each bf16 workload's shape at full size with an fp8 cache, through the
    one-call step the benchmark times with --kv-dtype fp8 (automatic kernel
    and split plan, fused append): codes, exponents and lengths bit-exact on
    the whole cache, attention against the oracle on every sequence or on a
    seeded sample of them."""
    w = inputs.WORKLOADS[name]
    say(f"fp8 full {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} T_cap={w.T_cap}")
    # drawn on the device (the cache is up to 1 GiB of codes per tensor)
    case = inputs.make_fp8_case(w.B, w.Hq, w.Hkv, w.D, w.T_cap, inputs.attended_lengths(w), seed=w.seed,
                                device="cuda")
    host = [t.cpu().numpy() for t in (case.k_codes, case.k_exp, case.v_codes, case.v_exp)]
    out, kc, ke, vc, ve, L, status, plan = fp8_step(case, w.Hq)
    say(f"fp8 full {name}: gpu done, plan={plan}, status={status}")
    assert status == kvd.KVD_OK
    f32 = lambda t: t.float().cpu().numpy()
    L0 = case.lengths0.cpu().numpy().astype(np.int32)
    kc2, ke2, vc2, ve2, L2, _ = oracle.append_fp8(*host, L0, f32(case.k_new), f32(case.v_new))
    assert np.array_equal(L.cpu().numpy(), L2)
    for got, want, what in ((kc, kc2, "K codes"), (ke, ke2, "K exponents"), (vc, vc2, "V codes"),
                            (ve, ve2, "V exponents")):
        assert np.array_equal(got.cpu().numpy(), want), what
    n = FP8_FULL[name]
    sel = np.arange(w.B) if n is None else np.sort(np.random.default_rng(w.seed).choice(w.B, n, replace=False))
    ref = oracle.decode_attention_fp8(f32(case.q)[sel], kc2[sel], ke2[sel], vc2[sel], ve2[sel], L2[sel], case.scale)
    err = rel_err_rows(to_f64(out)[sel], ref)
    say(f"fp8 full {name}: {len(sel)} sequences checked, max row-relative error {err:.3e}")
    assert err <= TOL_BF16, err


@pytest.mark.parametrize("name,T_q,page,sample", [("longctx_mqa_bf16", 4, 0, None), ("llama13b_mha_bf16", 8, 0, 8),
                                                  ("ragged_gqa_bf16", 1, 256, 16), ("longctx_mqa_bf16", 1, 256, None)])
def test_fp8_workload_full_size_multi_and_paged(name, T_q, page, sample):
    """The fp8 steps `bench.py --kv-dtype fp8` times with --new-tokens or
    --page-size, at full size: several new tokens (the append kernel, then
    the exchange or wave kernel over all query rows) and one new token on
    shuffled 256-token pages (fused append through the block table).
    Codes, exponents and lengths bit-exact on the whole cache; attention
    against the oracle on every sequence or a seeded sample."""
    w = inputs.WORKLOADS[name]
    say(f"fp8 full {name}: T_q={T_q} page={page}")
    case = inputs.make_fp8_case(w.B, w.Hq, w.Hkv, w.D, w.T_cap, inputs.attended_lengths(w), seed=w.seed + 5,
                                device="cuda", new_tokens=T_q if T_q > 1 else None)
    host = [t.cpu().numpy() for t in (case.k_codes, case.k_exp, case.v_codes, case.v_exp)]
    dev = torch.device("cuda")
    L = case.lengths0.to(dev, torch.int32, copy=True)
    if page:
        table, num_pages = inputs.paged_layout(w.B, w.T_cap, page, seed=w.seed)
        pools = [inputs.to_pages(x, table.to(x.device), page, num_pages).to(dev) for x in
                 (case.k_codes, case.k_exp, case.v_codes, case.v_exp)]
        bt = table.to(dev)
    else:
        pools = [x.to(dev, copy=True) for x in (case.k_codes, case.k_exp, case.v_codes, case.v_exp)]
        bt = None
    kc, ke, vc, ve = pools
    cache = kvd.KVCache(kc, vc, L, w.Hq, block_table=bt, k_exp=ke, v_exp=ve)
    try:
        plan = cache.plan()
        kn, vn, q = (t.contiguous() for t in (case.k_new, case.v_new, case.q))
        out = cache.step_multi(kn, vn, q, scale=case.scale) if T_q > 1 else cache.step(kn, vn, q, scale=case.scale)
        status = cache.status()
        torch.cuda.synchronize()
    finally:
        cache.close()
    say(f"fp8 full {name}: gpu done, plan={plan}, status={status}")
    assert status == kvd.KVD_OK
    got = [x.cpu().numpy() for x in (kc, ke, vc, ve)]
    if page:
        tb = table.numpy()
        got = [oracle.gather_pages(got[0], tb), oracle.gather_exponent_pages(got[1], tb),
               oracle.gather_pages(got[2], tb), oracle.gather_exponent_pages(got[3], tb)]
    f32 = lambda t: t.float().cpu().numpy()
    L0 = case.lengths0.cpu().numpy().astype(np.int32)
    if T_q > 1:
        kc2, ke2, vc2, ve2, L2, appended = oracle.append_fp8_multi(*host, L0, f32(case.k_new), f32(case.v_new))
    else:
        kc2, ke2, vc2, ve2, L2, _ = oracle.append_fp8(*host, L0, f32(case.k_new), f32(case.v_new))
    assert np.array_equal(L.cpu().numpy(), L2)
    for g, want, what in zip(got, (kc2, ke2, vc2, ve2), ("K codes", "K exponents", "V codes", "V exponents")):
        assert np.array_equal(g, want), what
    sel = np.arange(w.B) if sample is None else np.sort(np.random.default_rng(w.seed).choice(w.B, sample, replace=False))
    qs = f32(case.q)[sel]
    if T_q > 1:
        ref = oracle.decode_attention_fp8_multi(qs, kc2[sel], ke2[sel], vc2[sel], ve2[sel], L2[sel], appended[sel],
                                                case.scale)
    else:
        ref = oracle.decode_attention_fp8(qs, kc2[sel], ke2[sel], vc2[sel], ve2[sel], L2[sel], case.scale)
    err = rel_err_rows(to_f64(out)[sel], ref)
    say(f"fp8 full {name}: {len(sel)} sequences checked, max row-relative error {err:.3e}")
    assert err <= TOL_BF16, err


SHAPES = {  # name: (B, Hq, Hkv, D, T_cap, lengths)
    "palm_like": (3, 48, 1, 256, 2048, [2048, 1000, 33]),
    "mha_like": (2, 40, 40, 128, 4096, [4096, 1500]),
    "ragged_gqa_like": (8, 64, 8, 128, 8192, [64, 8192, 4000, 77, 1024, 5000, 31, 8000]),
    "long_mqa": (1, 48, 1, 256, 16384, [16384]),
    "small_d64": (2, 8, 1, 64, 160, [129, 64]),
    "gqa48_d128": (2, 96, 2, 128, 1024, [1000, 77]),     # three 16-row blocks per wave
    "gqa64_d128": (2, 64, 1, 128, 512, [500, 33]),       # two row groups (48 + 16)
}


@pytest.mark.parametrize("variant", ["wave", "lds", "xchg"])
@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name", list(SHAPES))
def test_fp8_shapes(name, fused, variant):
    B, Hq, Hkv, D, T, L = SHAPES[name]
    if variant in ("wave", "xchg") and D < 128:
        pytest.skip("the wave and exchange kernels need d >= 128")
    case = inputs.make_fp8_case(B, Hq, Hkv, D, T, L, seed=90 + len(name))
    check_fp8(case, Hq, f"fp8/{name}/{variant}", fused=fused, variant=variant)


@pytest.mark.parametrize("variant", ["wave", "lds", "xchg"])
@pytest.mark.parametrize("Hq", [16, 48])
@pytest.mark.parametrize("splits", [1, 2, 5])
def test_fp8_forced_splits(splits, Hq, variant):
    """Splits of 1 to 8 tiles: in the wave kernel some waves of a split get
    no tile at all, and lengths end on and next to tile edges."""
    lengths = [1, 31, 32, 33, 64, 65, 127, 128, 200, 256]
    case = inputs.make_fp8_case(len(lengths), Hq, 2, 128, 256, lengths, seed=95 + splits)
    check_fp8(case, Hq, f"fp8 S={splits} Hq={Hq} {variant}", splits=splits, variant=variant)


@pytest.mark.parametrize("Hq,Hkv,D", [(48, 1, 256), (32, 1, 256), (16, 2, 256), (96, 1, 256), (64, 1, 128),
                                     (80, 1, 128), (40, 2, 128)])
@pytest.mark.parametrize("splits", [None, 1, 3])
def test_fp8_xchg_row_groups_and_edges(Hq, Hkv, D, splits):
    """The exchange kernel over 1-4 row blocks per workgroup and several row
    groups (96 rows at d = 256: two groups of three blocks; 80 at d = 128:
    two groups of three), with lengths on and next to the edges of its
    16-token blocks and 64-token tiles, so that whole blocks of a tile lie
    past a sequence's end (lengths attended, the new token included: the
    fused append's token lands in slots 0, 16 and 64, opening a sequence, a
    block and a tile)."""
    lengths = [1, 15, 16, 17, 48, 63, 64, 65, 100, 129, 250]
    case = inputs.make_fp8_case(len(lengths), Hq, Hkv, D, 256, lengths, seed=150 + Hq + D)
    out, plan = check_fp8(case, Hq, f"fp8 xchg Hq={Hq} Hkv={Hkv} D={D} S={splits}", splits=splits,
                          variant="xchg")
    assert plan["variant"] == "xchg"


def test_fp8_append_extremes():
    """An all-zero row (exponent 0), a row needing a positive exponent, a
    row of tiny values and exact midpoints between codes."""
    B, Hq, Hkv, D, T = 4, 8, 2, 128, 64
    case = inputs.make_fp8_case(B, Hq, Hkv, D, T, [10, 20, 30, 40], seed=97)
    kn = case.k_new.float()
    kn[0, 0] = 0.0
    kn[1, 1] *= 5000.0
    kn[2, 0] *= 1e-6
    # midpoints of E4M3 neighbours, scaled so the row's maximum is exactly 448 * 2^-7
    kn[3, 0] = torch.tensor([1.0625, 1.1875, -1.0625, 448.0] * (D // 4)) * 2.0 ** -7
    case.k_new = kn.to(torch.bfloat16)
    case.v_new = (case.v_new.float() * 300.0).to(torch.bfloat16)
    check_fp8(case, Hq, "fp8 append extremes")


@pytest.mark.parametrize("variant", ["wave", "lds", "xchg"])
@pytest.mark.parametrize("k_e,v_e", [(-117, -117), (-6, -117), (-117, 64), (-4, 64)])
def test_fp8_exponent_range_edges(variant, k_e, v_e):
    """Every cached row at one exponent, at or near the ends of the stored
    range [-117, 119], over every finite code (subnormals included): keys at
    -117 score about 0 (uniform weights), values at -117 are the smallest
    normal bf16 numbers the format holds (weights times 2^-117), values at 64
    are large but keep the fp32 sums finite.  The kernels read code * 2^e
    exactly at either end."""
    B, Hq, Hkv, D, T = 2, 48, 1, 256, 256
    if variant == "lds" or variant == "wave":
        Hq = 16
    case = inputs.make_fp8_case(B, Hq, Hkv, D, T, [200, 77], seed=300 + k_e + v_e, k_exp_value=k_e,
                                v_exp_value=v_e)
    # the appended rows on the same scale (N(0,1) rows quantize to about 2^-7)
    case.k_new = (case.k_new.float() * 2.0 ** (k_e + 7)).to(torch.bfloat16)
    case.v_new = (case.v_new.float() * 2.0 ** (v_e + 7)).to(torch.bfloat16)
    check_fp8(case, Hq, f"fp8 exponent edge k_e={k_e} v_e={v_e} {variant}", variant=variant)


@pytest.mark.parametrize("fused", [True, False])
def test_fp8_append_exponent_clamp(fused):
    """New rows whose exponent falls outside the stored range: a row of
    values around 1e-36 takes exponent -117 (values below 2^-127 become 0), a
    row near bf16's largest value takes 119 and saturates at +-448; codes,
    exponents and lengths bit-exact against the oracle's append (through the
    separate append kernel, or the wave kernel's fused append)."""
    B, Hq, Hkv, D, T = 2, 8, 2, 128, 64
    case = inputs.make_fp8_case(B, Hq, Hkv, D, T, [10, 20], seed=310)
    kn = case.k_new.float()
    kn[0, 0] *= 1e-36
    kn[0, 1] = torch.linspace(-1.0, 1.0, D) * 3.3e38
    # largest 2^-109 gives exponent -117 exactly: 2^-126 becomes the smallest
    # code, 2^-128 rounds to 0, -2^-127 is a tie and goes to the even code -0
    kn[1, 0] = torch.tensor([2.0 ** -109, -(2.0 ** -127), 2.0 ** -128, 2.0 ** -126] * (D // 4))
    case.k_new = kn.to(torch.bfloat16)
    vn = case.v_new.float()
    vn[1, 1] *= 3e-38
    case.v_new = vn.to(torch.bfloat16)
    dev = torch.device("cuda")
    kc, vc = case.k_codes.to(dev, copy=True), case.v_codes.to(dev, copy=True)
    ke, ve = case.k_exp.to(dev, copy=True), case.v_exp.to(dev, copy=True)
    L = case.lengths0.to(dev, copy=True)
    cache = kvd.KVCache(kc, vc, L, Hq, k_exp=ke, v_exp=ve)
    try:
        cache.set_variant(kvd.KVD_VARIANT_WAVE)
        kn_d, vn_d = case.k_new.to(dev).contiguous(), case.v_new.to(dev).contiguous()
        if fused:
            # keys near bf16's largest value make some logits infinite: only
            # the cache is compared here
            cache.step(kn_d, vn_d, case.q.to(dev).contiguous(), scale=case.scale)
        else:
            cache.append(kn_d, vn_d)
        status = cache.status()
        torch.cuda.synchronize()
    finally:
        cache.close()
    assert status == kvd.KVD_OK
    f32 = lambda t: t.float().cpu().numpy()
    kc2, ke2, vc2, ve2, L2, _ = oracle.append_fp8(case.k_codes.numpy(), case.k_exp.numpy(), case.v_codes.numpy(),
                                                  case.v_exp.numpy(), case.lengths0.numpy().astype(np.int32),
                                                  f32(case.k_new), f32(case.v_new))
    assert ke2[0, 0, 9] == -117 and ke2[0, 1, 9] == 119, (ke2[0, 0, 9], ke2[0, 1, 9])
    assert ke2[1, 0, 19] == -117 and kc2[1, 0, 19, :4].tolist() == [0x78, 0x80, 0x00, 0x01]
    assert np.array_equal(L.cpu().numpy(), L2)
    for got, want, what in ((kc, kc2, "K codes"), (ke, ke2, "K exponents"), (vc, vc2, "V codes"),
                            (ve, ve2, "V exponents")):
        assert np.array_equal(got.cpu().numpy(), want), what


@pytest.mark.parametrize("name,B,Hq,Hkv,D,variant", [("mha", 2, 8, 8, 128, "wave"), ("gqa", 2, 64, 8, 128, "wave"),
                                                      ("mqa48_d128", 2, 48, 1, 128, "wave"),
                                                      ("mqa64_d128", 2, 64, 1, 128, "xchg"),
                                                      ("mqa48_d256", 2, 48, 1, 256, "xchg"),
                                                      ("mqa16_d256", 2, 16, 1, 256, "wave"),
                                                      ("d64", 2, 8, 1, 64, "lds")])
def test_fp8_auto_picks(name, B, Hq, Hkv, D, variant):
    """The automatic choice at d >= 128: the wave kernel when one workgroup
    holds the whole query group, else the exchange kernel; the shared-tile
    kernel at d = 64."""
    case = inputs.make_fp8_case(B, Hq, Hkv, D, 256, [200, 100], seed=77)
    out, plan = check_fp8(case, Hq, f"fp8 auto {name}")
    assert plan["variant"] == variant


def test_fp8_capacity_overflow():
    case = inputs.make_fp8_case(2, 8, 1, 128, 64, [64, 10], seed=98)
    L0 = torch.tensor([64, 9], dtype=torch.int32)
    out, kc, ke, vc, ve, L, status, plan = fp8_step(case, 8, lengths=L0)
    assert status == kvd.KVD_ECAPACITY
    assert L.cpu().tolist() == [64, 10]
    ref, kc2, ke2, vc2, ve2, L2 = oracle_fp8_step(case, lengths=L0)
    assert np.array_equal(kc.cpu().numpy(), kc2) and np.array_equal(ke.cpu().numpy(), ke2)
    assert rel_err_rows(to_f64(out), ref) <= TOL_BF16


@pytest.mark.parametrize("variant,Hq,D", [("wave", 16, 128), ("xchg", 48, 256), ("xchg", 64, 128)])
def test_fp8_fused_step_with_out_of_range_length(variant, Hq, D):
    """A length past capacity in a step whose append is fused into the wave
    or exchange kernel: no append for that sequence, attention clamped to
    capacity, KVD_ELENGTH; the other sequence steps normally."""
    case = inputs.make_fp8_case(2, Hq, 1, D, 96, [96, 41], seed=160)
    L_bad = torch.tensor([1000, 40], dtype=torch.int32)
    out, kc, ke, vc, ve, L, status, plan = fp8_step(case, Hq, lengths=L_bad, variant=variant)
    assert plan["variant"] == variant
    assert status == kvd.KVD_ELENGTH
    assert L.cpu().tolist() == [1000, 41]
    # sequence 0 is full in the oracle's run, so it is not appended there either
    ref, kc2, ke2, vc2, ve2, L2 = oracle_fp8_step(case, lengths=torch.tensor([96, 40], dtype=torch.int32))
    assert np.array_equal(kc.cpu().numpy(), kc2) and np.array_equal(ke.cpu().numpy(), ke2)
    assert np.array_equal(vc.cpu().numpy(), vc2) and np.array_equal(ve.cpu().numpy(), ve2)
    assert rel_err_rows(to_f64(out), ref) <= TOL_BF16


@pytest.mark.parametrize("variant", ["wave", "lds", "xchg"])
@pytest.mark.parametrize("phi", [0.0, -40.0, 1e4])
def test_fp8_unified_max(phi, variant):
    B, Hq, Hkv, D, T, L = SHAPES["palm_like"]
    case = inputs.make_fp8_case(B, Hq, Hkv, D, T, L, seed=99)
    check_fp8(case, Hq, f"fp8 unified max {phi} {variant}", unified_max=phi, variant=variant)


@pytest.mark.parametrize("variant", ["wave", "lds", "xchg"])
def test_fp8_consecutive_steps_ragged_batch(variant):
    """Several steps on one handle over a ragged batch: from the second step
    on the wave kernel dispatches sequences in the length order the previous
    combine sorted.  Each step's codes, exponents, lengths and output match
    the oracle run step by step."""
    B, Hq, Hkv, D, T, steps = 29, 64, 8, 128, 512, 3
    g = torch.Generator().manual_seed(123)
    L_att = torch.randint(1, T - steps, (B,), generator=g)
    case = inputs.make_fp8_case(B, Hq, Hkv, D, T, L_att.tolist(), seed=124)
    dev = torch.device("cuda")
    kc, vc = case.k_codes.to(dev, copy=True), case.v_codes.to(dev, copy=True)
    ke, ve = case.k_exp.to(dev, copy=True), case.v_exp.to(dev, copy=True)
    L = case.lengths0.to(dev, torch.int32, copy=True)
    cache = kvd.KVCache(kc, vc, L, Hq, k_exp=ke, v_exp=ve)
    cache.set_variant(VARIANTS[variant])
    r_kc, r_ke, r_vc, r_ve = (t.numpy() for t in (case.k_codes, case.k_exp, case.v_codes, case.v_exp))
    r_L = case.lengths0.numpy().astype(np.int32)
    try:
        for step in range(steps):
            gs = torch.Generator().manual_seed(500 + step)
            kn, vn = (torch.randn(B, Hkv, D, generator=gs).to(torch.bfloat16) for _ in range(2))
            q = torch.randn(B, Hq, D, generator=gs).to(torch.bfloat16)
            say(f"fp8 consecutive steps {variant}: step {step}")
            out = cache.step(kn.to(dev), vn.to(dev), q.to(dev), scale=D ** -0.5)
            r_kc, r_ke, r_vc, r_ve, r_L, _ = oracle.append_fp8(r_kc, r_ke, r_vc, r_ve, r_L, kn.float().numpy(),
                                                               vn.float().numpy())
            ref = oracle.decode_attention_fp8(q.float().numpy(), r_kc, r_ke, r_vc, r_ve, r_L, D ** -0.5)
            assert rel_err_rows(to_f64(out), ref) <= TOL_BF16, step
        assert cache.status() == kvd.KVD_OK
        torch.cuda.synchronize()
    finally:
        cache.close()
    assert np.array_equal(L.cpu().numpy(), r_L)
    assert np.array_equal(kc.cpu().numpy(), r_kc) and np.array_equal(ke.cpu().numpy(), r_ke)
    assert np.array_equal(vc.cpu().numpy(), r_vc) and np.array_equal(ve.cpu().numpy(), r_ve)


def fp8_paged_step(case, Hq, page_size, *, variant="wave", seed=5, fused=True, table_edit=None):
    """One step on fresh device copies of an fp8 case laid out in pages
    (codes and exponents under one seeded block table).  Returns (out,
    pools [kc, ke, vc, ve] after the step, pools before, table, lengths,
    status, plan)."""
    dev = torch.device("cuda")
    B, Hkv, T = case.k_codes.shape[:3]
    table, num_pages = inputs.paged_layout(B, T, page_size, seed)
    pools = [inputs.to_pages(x, table, page_size, num_pages) for x in (case.k_codes, case.k_exp, case.v_codes,
                                                                         case.v_exp)]
    before = [p.numpy().copy() for p in pools]
    kc, ke, vc, ve = (p.to(dev, copy=True) for p in pools)
    bt = table.clone()
    if table_edit is not None:  # the device's table only; the pools keep the layout of `table`
        table_edit(bt)
    bt = bt.to(dev)
    L = case.lengths0.to(dev, torch.int32, copy=True)
    cache = kvd.KVCache(kc, vc, L, Hq, block_table=bt, k_exp=ke, v_exp=ve)
    try:
        cache.set_variant(VARIANTS[variant])
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
    after = [t.cpu().numpy() for t in (kc, ke, vc, ve)]
    return out, after, before, table.numpy(), L.cpu().numpy(), status, plan


@pytest.mark.parametrize("variant", ["wave", "lds", "xchg"])
@pytest.mark.parametrize("name,page", [("ragged_gqa_like", 64), ("mha_like", 256), ("palm_like", 128),
                                       ("palm_like", 32), ("gqa48_d128", 32), ("small_d64", 32)])
def test_fp8_paged(name, page, variant):
    """fp8 codes and exponents in shuffled pages: the append (through the
    block table) is bit-exact on every pool, spare pages included, and the
    attention matches the oracle over the gathered cache."""
    B, Hq, Hkv, D, T, L = SHAPES[name]
    if variant in ("wave", "xchg") and D < 128:
        pytest.skip("the wave and exchange kernels need d >= 128")
    case = inputs.make_fp8_case(B, Hq, Hkv, D, T, L, seed=130 + len(name))
    say(f"fp8 paged {name} page={page} {variant}")
    out, after, before, bt, L_gpu, status, plan = fp8_paged_step(case, Hq, page, variant=variant)
    assert plan["variant"] == variant
    kc2, ke2, vc2, ve2, L2, _ = oracle.append_fp8_paged(*before, bt, case.lengths0.numpy(),
                                                        case.k_new.float().numpy(), case.v_new.float().numpy())
    assert status == kvd.KVD_OK
    assert np.array_equal(L_gpu, L2)
    for got, want, what in zip(after, (kc2, ke2, vc2, ve2), ("K codes", "K exponents", "V codes", "V exponents")):
        assert np.array_equal(got, want), what
    ref = oracle.decode_attention_fp8_paged(case.q.float().numpy(), kc2, ke2, vc2, ve2, bt, L2, case.scale)
    err = rel_err_rows(to_f64(out), ref)
    say(f"fp8 paged {name}: max row-relative error {err:.3e}")
    assert err <= TOL_BF16, err


def test_fp8_paged_equals_contiguous_bitwise():
    """Same plan, same arithmetic: the paged step's output equals the
    contiguous step's bit for bit."""
    B, Hq, Hkv, D, T, L = SHAPES["ragged_gqa_like"]
    case = inputs.make_fp8_case(B, Hq, Hkv, D, T, L, seed=140)
    out_c, *_ = fp8_step(case, Hq, variant="wave")
    out_p, *_ = fp8_paged_step(case, Hq, 64, variant="wave")
    assert torch.equal(out_c.cpu().view(torch.int16), out_p.cpu().view(torch.int16))


@pytest.mark.parametrize("variant", ["wave", "lds", "xchg"])
def test_fp8_paged_bad_entry_is_reported(variant):
    """A block-table entry in use outside the pool reads page 0 (memory
    safe) and is reported; the other sequences are unaffected."""
    case = inputs.make_fp8_case(2, 8, 1, 128, 128, [100, 70], seed=141)

    def corrupt(table):
        table[0, 1] = 10_000  # tokens 32..63 of sequence 0

    out, after, before, bt, L_gpu, status, plan = fp8_paged_step(case, 8, 32, variant=variant, table_edit=corrupt)
    assert status == kvd.KVD_EPAGE
    # (the table returned is the pools' layout; only sequence 0 read the bad entry)
    kc2, ke2, vc2, ve2, L2, _ = oracle.append_fp8_paged(*before, bt, case.lengths0.numpy(),
                                                        case.k_new.float().numpy(), case.v_new.float().numpy())
    ref = oracle.decode_attention_fp8_paged(case.q.float().numpy(), kc2, ke2, vc2, ve2, bt, L2, case.scale)
    assert rel_err_rows(to_f64(out)[1:], ref[1:]) <= TOL_BF16


def fp8_multi_check(B, Hq, Hkv, D, T, L_att, T_q, name, *, variant="auto", splits=None, page=0,
                    expect=kvd.KVD_OK):
    """Several new tokens per sequence on an fp8 cache (contiguous or paged):
    the quantizing append of all T_q rows is bit-exact and query i attends
    over the cache and new tokens 0..i, against the oracle."""
    case = inputs.make_fp8_case(B, Hq, Hkv, D, T, L_att, seed=200 + T_q + D + page)
    g = torch.Generator().manual_seed(300 + T_q)
    kn, vn = (torch.randn(B, Hkv, T_q, D, generator=g).to(torch.bfloat16) for _ in range(2))
    q = torch.randn(B, Hq, T_q, D, generator=g).to(torch.bfloat16)
    say(f"fp8 multi {name}: B={B} Hq={Hq} Hkv={Hkv} D={D} T_q={T_q} page={page} {variant} S={splits}")
    dev = torch.device("cuda")
    host = [case.k_codes, case.k_exp, case.v_codes, case.v_exp]
    if page:
        table, num_pages = inputs.paged_layout(B, T, page, seed=7)
        host = [inputs.to_pages(x, table, page, num_pages) for x in host]
    kc, ke, vc, ve = (x.to(dev, copy=True) for x in host)
    L = case.lengths0.to(dev, torch.int32, copy=True)
    bt = table.to(dev) if page else None
    cache = kvd.KVCache(kc, vc, L, Hq, block_table=bt, k_exp=ke, v_exp=ve)
    try:
        cache.set_variant(VARIANTS[variant])
        if splits is not None:
            cache.set_num_splits(splits)
        out = cache.step_multi(kn.to(dev), vn.to(dev), q.to(dev), scale=D ** -0.5)
        status = cache.status()
        torch.cuda.synchronize()
    finally:
        cache.close()
    assert status == expect
    before = [x.numpy() for x in host]
    if page:
        gather = [oracle.gather_pages(before[0], table.numpy()), oracle.gather_exponent_pages(before[1], table.numpy()),
                  oracle.gather_pages(before[2], table.numpy()), oracle.gather_exponent_pages(before[3], table.numpy())]
    else:
        gather = before
    r_kc, r_ke, r_vc, r_ve, r_L, appended = oracle.append_fp8_multi(*gather, case.lengths0.numpy(),
                                                                     kn.float().numpy(), vn.float().numpy())
    assert np.array_equal(L.cpu().numpy(), r_L)
    got = [x.cpu().numpy() for x in (kc, ke, vc, ve)]
    if page:
        got = [oracle.gather_pages(got[0], table.numpy()), oracle.gather_exponent_pages(got[1], table.numpy()),
               oracle.gather_pages(got[2], table.numpy()), oracle.gather_exponent_pages(got[3], table.numpy())]
    for a, b, what in zip(got, (r_kc, r_ke, r_vc, r_ve), ("K codes", "K exponents", "V codes", "V exponents")):
        assert np.array_equal(a, b), what
    ref = oracle.decode_attention_fp8_multi(q.float().numpy(), r_kc, r_ke, r_vc, r_ve, r_L, appended, D ** -0.5)
    err = rel_err_rows(to_f64(out).reshape(-1, D), ref.reshape(-1, D))
    say(f"fp8 multi {name}: max row-relative error {err:.3e}")
    assert err <= TOL_BF16, err


@pytest.mark.parametrize("variant", ["wave", "lds", "xchg"])
@pytest.mark.parametrize("shape,T_q", [("mha", 4), ("gqa", 4), ("gqa", 8), ("palm_like", 2), ("gqa_d256", 3)])
def test_fp8_multi_token(shape, T_q, variant):
    B, Hq, Hkv, D, T, L = {
        "mha": (2, 16, 16, 128, 512, [400, 95]),
        "gqa": (4, 64, 8, 128, 1024, [1000, 1, 33, 513]),
        "palm_like": (3, 48, 1, 256, 2048, [2000, 31, 700]),
        "gqa_d256": (2, 32, 4, 256, 512, [300, 64]),
    }[shape]
    fp8_multi_check(B, Hq, Hkv, D, T, L, T_q, f"{shape} T_q={T_q}", variant=variant)


@pytest.mark.parametrize("variant", ["wave", "lds", "xchg"])
@pytest.mark.parametrize("splits", [1, 3, 9])
def test_fp8_multi_token_empty_splits(variant, splits):
    """Lengths just below tile edges: early queries' last tokens end in
    tiles (and waves and splits) that the later queries reach past."""
    fp8_multi_check(5, 16, 2, 128, 256, [31, 60, 95, 1, 64], 6, f"edges S={splits}", variant=variant,
                    splits=splits)


def test_fp8_multi_token_paged_and_overflow():
    fp8_multi_check(3, 48, 1, 256, 512, [200, 33, 480], 4, "paged", page=64)
    fp8_multi_check(3, 16, 2, 128, 128, [126, 124, 10], 4, "overflow", expect=kvd.KVD_ECAPACITY)


def test_fp8_maximum_capacity():
    """The largest fp8 cache the header accepts, 2^24 tokens (one sequence,
    8 heads, d = 64, 1 GiB of codes per tensor): one fused step appends
    slot 2^24 - 1 and attends every token; codes, exponents and lengths
    bit for bit, all heads against the oracle."""
    T = 1 << 24
    case = inputs.make_fp8_case(1, 8, 1, 64, T, torch.tensor([T], dtype=torch.int32), seed=2424, device="cuda")
    say("fp8 maximum capacity: B=1 Hq=8 Hkv=1 D=64 T=2^24")
    out, kc, ke, vc, ve, L, status, plan = fp8_step(case, 8)
    say(f"fp8 maximum capacity: gpu done, plan={plan}, status={status}")
    assert status == kvd.KVD_OK
    host = lambda t: t.cpu().numpy()
    f32 = lambda t: t.float().cpu().numpy()
    L0 = case.lengths0.cpu().numpy().astype(np.int32)
    kc2, ke2, vc2, ve2, L2, _ = oracle.append_fp8(host(case.k_codes), host(case.k_exp), host(case.v_codes),
                                                  host(case.v_exp), L0, f32(case.k_new), f32(case.v_new))
    assert np.array_equal(L.cpu().numpy(), L2)
    for got, want, what in ((kc, kc2, "K codes"), (ke, ke2, "K exponents"), (vc, vc2, "V codes"),
                            (ve, ve2, "V exponents")):
        assert np.array_equal(host(got), want), what
    del kc, vc
    ref = oracle.decode_attention_fp8(f32(case.q), kc2, ke2, vc2, ve2, L2, case.scale)
    err = rel_err_rows(to_f64(out), ref)
    say(f"fp8 maximum capacity: max row-relative error {err:.3e}")
    assert err <= TOL_BF16, err
    torch.cuda.empty_cache()


def test_fp8_cache_past_4_gib():
    """An fp8 MHA cache of 5.4 GB of codes per tensor (128 sequences, 40 KV
    heads, 8192 tokens, d = 128): code offsets of the later sequences pass
    2^32.  One fused step on the automatic plan; the first, a middle and the
    last sequence are checked against the oracle on their own slices."""
    B, H, T, D = 128, 40, 8192, 128
    L_att = torch.full((B,), T, dtype=torch.int32)
    L_att[1::2] = T - 100
    case = inputs.make_fp8_case(B, H, H, D, T, L_att, seed=4322, device="cuda")
    assert case.k_codes.numel() > 2 ** 32
    picks = [0, B // 2, B - 1]
    sl = lambda t, b: t[b:b + 1].cpu().numpy()
    before = {b: [sl(t, b) for t in (case.k_codes, case.k_exp, case.v_codes, case.v_exp)] for b in picks}
    say(f"fp8 cache past 4 GiB: B={B} H={H} T={T} D={D}")
    out, kc, ke, vc, ve, L, status, plan = fp8_step(case, H)
    say(f"fp8 cache past 4 GiB: gpu done, plan={plan}, status={status}")
    assert status == kvd.KVD_OK
    L0 = case.lengths0.cpu().numpy().astype(np.int32)
    assert np.array_equal(L.cpu().numpy(), L0 + 1)
    f32 = lambda t, b: t[b:b + 1].float().cpu().numpy()
    for b in picks:
        kc2, ke2, vc2, ve2, L2, _ = oracle.append_fp8(*before[b], L0[b:b + 1], f32(case.k_new, b), f32(case.v_new, b))
        for got, want, what in ((kc, kc2, "K codes"), (ke, ke2, "K exponents"), (vc, vc2, "V codes"),
                                (ve, ve2, "V exponents")):
            assert np.array_equal(sl(got, b), want), (what, b)
        ref = oracle.decode_attention_fp8(f32(case.q, b), kc2, ke2, vc2, ve2, L2, case.scale)
        err = rel_err_rows(to_f64(out[b:b + 1]), ref)
        say(f"fp8 cache past 4 GiB: sequence {b} max row-relative error {err:.3e}")
        assert err <= TOL_BF16, err
    del case, out, kc, ke, vc, ve
    torch.cuda.empty_cache()  # return the 22 GB to the device for the tests after this one
