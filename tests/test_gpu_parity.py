"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every workload runs at full size (the launch configuration the benchmark
times, automatic split plan) and is compared element by element with the
fp64 oracle on the same bytes; reduced-batch variants, forced split counts,
both partial-pass kernels and the degenerate cases run at sizes that still
span several tiles and a ragged tail.
"""
import math

import numpy as np
import pytest
import torch

import multiquery_decode_attention_amd as kvd
from multiquery_decode_attention_amd import inputs
from conftest import TOL_BF16, TOL_F32, rel_err_rows
import oracle
from gpu_helpers import gpu_step, oracle_step, say, to_f64

pytestmark = pytest.mark.gpu


def tol_for(case):
    return TOL_BF16 if case.q.dtype == torch.bfloat16 else TOL_F32


def check_case(case, Hq, name, **kw):
    say(f"{name}: B={case.q.shape[0]} Hq={Hq} Hkv={case.k_cache.shape[1]} "
        f"T_cap={case.k_cache.shape[2]} D={case.q.shape[2]} dtype={case.q.dtype} {kw}")
    out, kc, vc, L, status, plan = gpu_step(case, Hq, **kw)
    say(f"{name}: gpu done, plan={plan}, status={status}")
    ref, k2, v2, L2 = oracle_step(case, lengths=kw.get("lengths"))
    assert status == kvd.KVD_OK
    # append: bit-exact on the whole cache and on the lengths
    assert np.array_equal(L.cpu().numpy(), L2)
    assert np.array_equal(inputs.host_array(kc), k2), "K cache differs after append"
    assert np.array_equal(inputs.host_array(vc), v2), "V cache differs after append"
    err = rel_err_rows(to_f64(out), ref)
    say(f"{name}: max row-relative error {err:.3e} (tol {tol_for(case):.0e})")
    assert err <= tol_for(case), err
    return out, ref, plan


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_workload_full_size(name):
    """Each named workload at its full size, all outputs checked, through
    the one-call step (kvdecode_append_attend) the benchmark times and
    through separate append and attend calls."""
    w = inputs.WORKLOADS[name]
    case = inputs.make_workload_case(w, device="cuda")
    check_case(case, w.Hq, name, fused=True)
    check_case(case, w.Hq, name + "/separate")


@pytest.mark.parametrize("variant", ["lds", "mfma", "valu"])
@pytest.mark.parametrize("splits", [0, 1, 5])
def test_fused_step_matches_oracle(variant, splits):
    """kvdecode_append_attend == append then attend: ragged lengths whose
    new token lands on every position of a tile, at tile edges, and in
    splits other than the first."""
    lengths = [1, 2, 31, 32, 33, 63, 64, 65, 96, 100, 127, 128, 129, 200]
    for dtype in (["bf16"] if variant != "valu" else ["bf16", "f32"]):
        case = inputs.make_case(len(lengths), 48, 2, 128, 200, lengths, dtype, seed=77 + splits)
        check_case(case, 48, f"fused {variant} splits={splits} {dtype}", fused=True,
                   variant=VARIANTS[variant], splits=splits)


@pytest.mark.parametrize("name,B", [("palm_mqa_bf16", 3), ("llama13b_mha_bf16", 2),
                                    ("ragged_gqa_bf16", 6), ("tiny_mqa_f32", 1)])
@pytest.mark.parametrize("splits", [1, 2, 7, 0])
def test_split_invariance(name, B, splits):
    """Any split count gives the oracle's answer (the LSE merge is exact
    algebra; only rounding order changes)."""
    w = inputs.WORKLOADS[name]
    case = inputs.make_workload_case(w, device="cpu", B=B)
    check_case(case, w.Hq, f"{name}/splits={splits}", splits=splits)


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("splits", [17, 24, 33, 50, 64])
def test_many_splits_d256(splits, fused):
    """d = 256 bf16 rows over 17..64 splits (the combine's split groups meet
    in LDS): ragged lengths with a sequence of one token, one shorter than
    the split count in tiles, and a full one, every row against the
    oracle."""
    lengths = [1, 20 * 32 + 5, 2048, 1500]
    case = inputs.make_case(len(lengths), 48, 1, 256, 2048, lengths, "bf16", seed=300 + splits)
    check_case(case, 48, f"many splits {splits} fused={fused}", splits=splits, fused=fused)


@pytest.mark.parametrize("variant", ["valu"])
def test_bf16_cache_past_4_gib(variant):
    """test_cache_past_4_gib on the vector-ALU kernel: a bf16 MHA cache of
    5.4 GB per tensor (64 sequences, 40 KV heads, 8192 tokens, d = 128),
    whose later sequences' byte offsets pass 2^32 in the fused append, the
    partial pass and the combine; the first, a middle and the last sequence
    against the oracle on their own slices (the append bit for bit)."""
    B, H, T, D = 64, 40, 8192, 128
    L_att = torch.full((B,), T, dtype=torch.int32)
    L_att[1::2] = T - 100
    case = inputs.make_case(B, H, H, D, T, L_att, "bf16", seed=4323, device="cuda")
    assert case.k_cache.numel() * 2 > 2 ** 32
    picks = [0, B // 2, B - 1]
    sl = lambda t, b: inputs.host_array(t[b:b + 1])
    before = {b: (sl(case.k_cache, b), sl(case.v_cache, b)) for b in picks}
    say(f"bf16 cache past 4 GiB ({variant}): B={B} H={H} T={T} D={D}")
    out, kc, vc, L, status, plan = gpu_step(case, H, variant=VARIANTS[variant], fused=True)
    say(f"bf16 cache past 4 GiB ({variant}): gpu done, plan={plan}, status={status}")
    assert status == kvd.KVD_OK
    L0 = case.lengths0.cpu().numpy().astype(np.int32)
    assert np.array_equal(L.cpu().numpy(), L0 + 1)
    for b in picks:
        k2, v2, L2, _ = oracle.append(*before[b], L0[b:b + 1], sl(case.k_new, b), sl(case.v_new, b))
        assert np.array_equal(sl(kc, b), k2) and np.array_equal(sl(vc, b), v2), b
        ref = oracle.decode_attention(sl(case.q, b), k2, v2, L2, case.scale, oracle.BF16)
        err = rel_err_rows(to_f64(out[b:b + 1]), ref)
        say(f"bf16 cache past 4 GiB ({variant}): sequence {b} max row-relative error {err:.3e}")
        assert err <= TOL_BF16, err
    del case, out, kc, vc
    torch.cuda.empty_cache()


VARIANTS = {"auto": kvd.KVD_VARIANT_AUTO, "valu": kvd.KVD_VARIANT_VALU, "mfma": kvd.KVD_VARIANT_MFMA, "lds": kvd.KVD_VARIANT_LDS}


@pytest.mark.parametrize("variant", ["valu", "mfma", "lds"])
@pytest.mark.parametrize("name,B", [("palm_mqa_bf16", 2), ("ragged_gqa_bf16", 4),
                                    ("llama13b_mha_bf16", 1), ("longctx_mqa_bf16", 1)])
def test_kernel_variants_bf16(name, B, variant):
    """Each partial-pass kernel on its own (the vector-ALU one is an
    independent second GPU path)."""
    w = inputs.WORKLOADS[name]
    case = inputs.make_workload_case(w, device="cpu", B=B)
    if name == "longctx_mqa_bf16":  # keep the CPU copy small: 8192 tokens
        case = inputs.make_case(1, w.Hq, w.Hkv, w.D, 8192, [8192], "bf16", seed=w.seed)
    check_case(case, w.Hq, f"{name}/{variant}", variant=VARIANTS[variant])


@pytest.mark.parametrize("dtype,variant", [("bf16", "lds"), ("bf16", "mfma"), ("f32", "valu")])
@pytest.mark.parametrize("Hq,Hkv,D", [(48, 1, 256), (8, 1, 64), (64, 8, 128), (12, 4, 128),
                                      (80, 1, 128), (16, 16, 64), (17, 1, 256), (130, 2, 64)])
def test_shapes_and_ragged_lengths(dtype, variant, Hq, Hkv, D):
    """Group sizes 1..65 (one to five 16-head blocks, one or two 64-head
    groups, padded ones too), every head dim, and lengths hitting 1, tile
    edges and capacity, with a forced split count that cuts mid-sequence."""
    T_cap = 300
    lengths = [1, 2, 31, 32, 33, 64, 65, 257, 300]  # attended lengths (after append)
    B = len(lengths)
    case = inputs.make_case(B, Hq, Hkv, D, T_cap, lengths, dtype, seed=Hq * 1000 + D, device="cpu")
    for splits in (0, 3):
        check_case(case, Hq, f"shape Hq={Hq} Hkv={Hkv} D={D} {dtype} {variant} splits={splits}",
                   variant=VARIANTS[variant], splits=splits)


@pytest.mark.parametrize("splits", [0, 2])
@pytest.mark.parametrize("variant", ["lds", "valu"])
def test_maximum_batch(variant, splits):
    """The largest batch the header accepts, 65535 sequences (8 heads, one
    KV head, d = 64, capacity 128, ragged lengths 1..128 after the append):
    the automatic one-split plan (per-sequence arrival counters for every
    sequence) and two splits (the combine over all of them, past its
    2048-sequence sort).  Fused step; every row against the oracle, the
    append bit for bit."""
    B, T = 65535, 128
    lengths = torch.randint(1, T + 1, (B,), generator=torch.Generator().manual_seed(65535), dtype=torch.int32)
    case = inputs.make_case(B, 8, 1, 64, T, lengths, "bf16", seed=65535)
    check_case(case, 8, f"maximum batch {variant} splits={splits}", fused=True,
               variant=VARIANTS[variant], splits=splits)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_maximum_capacity(dtype):
    """The largest cache the header accepts, 2^24 tokens (one sequence,
    d = 64; 2 GiB per tensor in bf16, 4 GiB in fp32): the fused step
    appends slot 2^24 - 1 and attends every token; all 8 heads against the
    oracle, the append bit for bit on the whole cache."""
    T = 1 << 24
    case = inputs.make_case(1, 8, 1, 64, T, [T], dtype, seed=24, device="cuda")
    _, _, plan = check_case(case, 8, f"maximum capacity {dtype}", fused=True)
    assert plan["num_splits"] * plan["split_tokens"] >= T
    del case
    torch.cuda.empty_cache()


@pytest.mark.parametrize("splits", [None, 1])
def test_empty_sequences_and_poisoned_tails(splits):
    """len 0 gives a zero row; slots past the length hold NaN/Inf and must
    never reach the output.  With one split the partial pass writes the
    output itself, zero rows included."""
    B, Hq, Hkv, D, T_cap = 5, 48, 1, 256, 200
    case = inputs.make_case(B, Hq, Hkv, D, T_cap, [1, 1, 50, 199, 200], "bf16", seed=7)
    L0 = torch.tensor([0, 0, 49, 198, 199], dtype=torch.int32)
    for b, n in enumerate(L0.tolist()):
        case.k_cache[b, :, n + 1:] = float("nan")
        case.v_cache[b, :, n + 1:] = float("inf")
    # sequences 0 and 1: attend without appending -> one empty, checked below
    out, _, _, L, status, _ = gpu_step(case, Hq, append=False, lengths=L0, splits=splits)
    assert status == kvd.KVD_OK
    ref, _, _, _ = oracle_step(case, append=False, lengths=L0)
    o = to_f64(out)
    assert np.all(o[0] == 0) and np.all(o[1] == 0)
    assert rel_err_rows(o, ref) <= TOL_BF16
    # with the append every sequence is non-empty
    check_case(case, Hq, f"poisoned tails + append, splits={splits}", lengths=L0, splits=splits)
    check_case(case, Hq, f"poisoned tails + fused append, splits={splits}", lengths=L0, splits=splits, fused=True)


@pytest.mark.parametrize("fused,variant", [(False, "auto"), (True, "lds"), (True, "valu"), (True, "mfma")])
def test_capacity_overflow_reported_and_harmless(fused, variant):
    B, Hq, Hkv, D, T_cap = 3, 8, 2, 128, 64
    case = inputs.make_case(B, Hq, Hkv, D, T_cap, [64, 64, 10], "bf16", seed=9)
    L0 = torch.tensor([64, 63, 9], dtype=torch.int32)  # sequence 0 is already full
    out, kc, vc, L, status, _ = gpu_step(case, Hq, lengths=L0, fused=fused, variant=VARIANTS[variant])
    assert status == kvd.KVD_ECAPACITY
    assert L.cpu().tolist() == [64, 64, 10]
    ref, k2, v2, L2 = oracle_step(case, lengths=L0)
    assert L2.tolist() == [64, 64, 10]
    assert np.array_equal(inputs.host_array(kc), k2) and np.array_equal(inputs.host_array(vc), v2)
    assert rel_err_rows(to_f64(out), ref) <= TOL_BF16


@pytest.mark.parametrize("variant,fused", [("lds", True), ("valu", True), ("mfma", False)])
def test_reserve_then_step(variant, fused):
    """kvdecode_reserve before the first call changes no result."""
    case = inputs.make_case(3, 16, 2, 128, 200, [1, 77, 199], "bf16", seed=31)
    check_case(case, 16, f"reserve {variant}", variant=VARIANTS[variant], fused=fused, reserve=True)


@pytest.mark.parametrize("variant", ["lds", "valu"])
def test_fused_step_with_out_of_range_length(variant):
    """A length past capacity: no append for that sequence, attention
    clamped to capacity, KVD_ELENGTH; the other sequence steps normally."""
    B, Hq, Hkv, D, T_cap = 2, 16, 1, 128, 96
    case = inputs.make_case(B, Hq, Hkv, D, T_cap, [96, 41], "bf16", seed=12)
    L_bad = torch.tensor([1000, 40], dtype=torch.int32)
    out, kc, vc, L, status, _ = gpu_step(case, Hq, lengths=L_bad, fused=True, variant=VARIANTS[variant])
    assert status == kvd.KVD_ELENGTH
    assert L.cpu().tolist() == [1000, 41]
    ref, k2, v2, _ = oracle_step(case, lengths=torch.tensor([96, 40], dtype=torch.int32))
    # sequence 0 is full in the oracle's run, so it is not appended there either
    assert np.array_equal(inputs.host_array(kc), k2) and np.array_equal(inputs.host_array(vc), v2)
    assert rel_err_rows(to_f64(out), ref) <= TOL_BF16


@pytest.mark.parametrize("dtype,variant", [("bf16", "lds"), ("bf16", "mfma"), ("f32", "valu")])
def test_separate_append_with_out_of_range_length(dtype, variant):
    """The separate append (kvdecode_append, and the append kernel the MFMA
    step runs first) on a length past capacity reports it as a bad length,
    KVD_ELENGTH, as the fused step does -- not as a full cache -- and leaves
    that sequence unchanged; the other sequence is appended."""
    B, Hq, Hkv, D, T_cap = 2, 16, 1, 128, 96
    case = inputs.make_case(B, Hq, Hkv, D, T_cap, [96, 41], dtype, seed=13)
    L_bad = torch.tensor([1000, 40], dtype=torch.int32)
    out, kc, vc, L, status, _ = gpu_step(case, Hq, lengths=L_bad, fused=False, variant=VARIANTS[variant])
    assert status == kvd.KVD_ELENGTH
    assert L.cpu().tolist() == [1000, 41]
    ref, k2, v2, _ = oracle_step(case, lengths=torch.tensor([96, 40], dtype=torch.int32))
    assert np.array_equal(inputs.host_array(kc), k2) and np.array_equal(inputs.host_array(vc), v2)
    assert rel_err_rows(to_f64(out), ref) <= tol_for(case)


def test_length_out_of_range_is_clamped_and_reported():
    B, Hq, Hkv, D, T_cap = 2, 16, 1, 128, 96
    case = inputs.make_case(B, Hq, Hkv, D, T_cap, [96, 40], "bf16", seed=10)
    L_bad = torch.tensor([1000, 40], dtype=torch.int32)
    out, _, _, _, status, _ = gpu_step(case, Hq, append=False, lengths=L_bad)
    assert status == kvd.KVD_ELENGTH
    ref, _, _, _ = oracle_step(case, append=False, lengths=torch.tensor([96, 40], dtype=torch.int32))
    assert rel_err_rows(to_f64(out), ref) <= TOL_BF16


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hand_worked_cases_on_gpu(dtype):
    """The exact hand-worked fixtures, zero-padded from d=2/4 to d=64 (zero
    columns change no dot product and give zero output columns)."""
    import json
    from fractions import Fraction
    from oracle_pins import GOLDEN
    for c in json.load(open(GOLDEN))["cases"]:
        B, Hq, Hkv, d, T = c["B"], c["Hq"], c["Hkv"], c["D"], c["T_cap"]
        D = 64
        tdt = torch.float32 if dtype == "f32" else torch.bfloat16
        def pad(x, shape):
            z = torch.zeros(shape, dtype=torch.float32)
            z[..., :d] = torch.tensor(x, dtype=torch.float32)
            return z.to(tdt)
        q = pad(c["q"], (B, Hq, D))
        k = pad(c["k"], (B, Hkv, T, D))
        v = pad(c["v"], (B, Hkv, T, D))
        L = torch.tensor(c["lengths"], dtype=torch.int32)
        if c.get("poison_tail"):
            for b, n in enumerate(L.tolist()):
                k[b, :, n:] = float("nan")
                v[b, :, n:] = float("nan")
        scale = eval(c["scale_expr"], {"log": math.log})  # noqa: S307 (fixture-owned)
        case = inputs.Case(q, k, v, L, torch.zeros(B, Hkv, D, dtype=tdt),
                           torch.zeros(B, Hkv, D, dtype=tdt), scale)
        for variant in ([kvd.KVD_VARIANT_VALU] +
                        ([kvd.KVD_VARIANT_MFMA, kvd.KVD_VARIANT_LDS] if dtype == "bf16" else [])):
            out, _, _, _, status, _ = gpu_step(case, Hq, append=False, variant=variant)
            assert status == kvd.KVD_OK
            got = to_f64(out)[..., :d]
            want = np.array([[[float(Fraction(x)) for x in r] for r in hb] for hb in c["out"]])
            tol = TOL_F32 if dtype == "f32" else TOL_BF16
            assert rel_err_rows(got, want) <= tol, (c["id"], variant, got, want)
            assert np.all(to_f64(out)[..., d:] == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cached_decode_equals_naive_recompute(dtype):
    """Start from an empty cache; at every step append the token's K/V and
    attend its query.  Row i must equal full causal attention recomputed
    from scratch over tokens 0..i ("All About Transformer Inference",
    section "Transformer inference basics")."""
    torch.manual_seed(5)
    T, E, Hq, Hkv, D = 70, 96, 16, 2, 128
    M = Hq // Hkv
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    x = torch.randn(T, E, dtype=torch.float64)
    Wq, Wk, Wv = (torch.randn(E, n * D, dtype=torch.float64) / math.sqrt(E) for n in (Hq, Hkv, Hkv))
    Q = (x @ Wq).view(T, Hq, D).to(tdt)
    K = (x @ Wk).view(T, Hkv, D).to(tdt)
    V = (x @ Wv).view(T, Hkv, D).to(tdt)
    scale = D ** -0.5
    # from scratch, fp64 on the CPU, on the cache-dtype values
    Qd, Kd, Vd = Q.double(), K.double(), V.double()
    full = torch.zeros(T, Hq, D, dtype=torch.float64)
    mask = torch.tril(torch.ones(T, T, dtype=torch.bool))
    for h in range(Hq):
        S = scale * (Qd[:, h] @ Kd[:, h // M].T)
        S = S.masked_fill(~mask, float("-inf"))
        full[:, h] = torch.softmax(S, dim=1) @ Vd[:, h // M]
    # cached, on the GPU
    dev = torch.device("cuda")
    kc = torch.full((1, Hkv, T, D), float("nan"), dtype=tdt, device=dev)
    vc = torch.full((1, Hkv, T, D), float("nan"), dtype=tdt, device=dev)
    L = torch.zeros(1, dtype=torch.int32, device=dev)
    cache = kvd.KVCache(kc, vc, L, Hq)
    rows = []
    for i in range(T):
        kn, vn, qi = (X[i][None].to(dev).contiguous() for X in (K, V, Q))
        if i % 2:  # alternate the one-call step and separate calls
            rows.append(cache.step(kn, vn, qi, scale=scale))
        else:
            cache.append(kn, vn)
            rows.append(cache.attend(qi, scale=scale))
    assert cache.status() == kvd.KVD_OK
    cache.close()
    got = torch.cat(rows).double().cpu().numpy()
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert rel_err_rows(got, full.numpy()) <= tol
    assert L.item() == T


@pytest.mark.parametrize("phi", [None, 0.0, 6.0, -40.0, 200.0, 1e4])
@pytest.mark.parametrize("name,B", [("palm_mqa_bf16", 2), ("ragged_gqa_bf16", 4), ("longctx_mqa_bf16", 1)])
def test_unified_max_any_bound_same_result(name, B, phi):
    """Asynchronous softmax with a unified maximum: a bound near the logits,
    far below them (every split raises it), far above them (every split
    starts from its own maximum) -- the oracle's result every time, through
    the long-split and short-split LDS configurations."""
    w = inputs.WORKLOADS[name]
    case = inputs.make_workload_case(w, device="cpu", B=B)
    if name == "longctx_mqa_bf16":
        case = inputs.make_case(1, w.Hq, w.Hkv, w.D, 16384, [16384], "bf16", seed=w.seed)
    check_case(case, w.Hq, f"{name} unified max {phi}", fused=True, unified_max=phi)


@pytest.mark.parametrize("splits", [4, 1])
@pytest.mark.parametrize("what", ["all", "partial"])
def test_timing_brackets(what, splits):
    """Event timing records only the brackets asked for and leaves results
    unchanged: timed steps equal untimed ones bit for bit.  The timed
    launches stamp their own events: a one-split pass launches no combine,
    so its combine bracket is exactly zero."""
    case = inputs.make_case(2, 16, 2, 128, 300, [100, 250], "bf16", seed=41)
    dev = torch.device("cuda")
    mask = kvd.KVD_TIME_ALL if what == "all" else kvd.KVD_TIME_PARTIAL
    outs, timings = [], []
    for timed in (False, True):
        kc, vc = case.k_cache.to(dev, copy=True), case.v_cache.to(dev, copy=True)
        L = case.lengths0.to(dev, torch.int32, copy=True)
        cache = kvd.KVCache(kc, vc, L, 16)
        try:
            cache.set_variant(VARIANTS["lds"])
            cache.set_num_splits(splits)
            if timed:
                kvd.kvdecode_timing_enable(cache.handle, 3, mask)
            kn, vn, q = (t.to(dev) for t in (case.k_new, case.v_new, case.q))
            outs.append(cache.step(kn, vn, q, scale=case.scale))
            cache.append(kn, vn)  # separate append, then attend
            outs.append(cache.attend(q, scale=case.scale))
            torch.cuda.synchronize()
            if timed:
                timings.append(kvd.kvdecode_timing_read(cache.handle))
        finally:
            cache.close()
    say(f"timing {what}: {timings}")
    assert torch.equal(outs[0].view(torch.int16), outs[2].view(torch.int16))
    assert torch.equal(outs[1].view(torch.int16), outs[3].view(torch.int16))
    t = timings[0]
    assert t["n_attend"] == 2 and t["partial_ms"] > 0
    if what == "all":
        assert (t["combine_ms"] > 0) == (splits > 1) and t["append_ms"] > 0 and t["n_append"] == 1
    else:
        assert t["combine_ms"] == 0 and t["append_ms"] == 0 and t["n_append"] == 0


@pytest.mark.parametrize("splits", [0, 1])
@pytest.mark.parametrize("variant", ["lds", "valu"])
@pytest.mark.parametrize("Hq,Hkv,D", [(16, 2, 128), (96, 1, 256)])
def test_consecutive_steps_ragged_batch(variant, Hq, Hkv, D, splits):
    """Several steps on one handle over a ragged batch.  From the second
    step on, the LDS kernel dispatches the sequences in the length order the
    previous combine sorted (and 96 heads take two head groups); every
    step's output and appended cache must match the oracle run step by
    step.  With one split there is no combine: the last of each sequence's
    workgroups advances its length, counted on a per-sequence counter that
    every step must leave at zero for the next."""
    B, T_cap, steps = 37, 512, 4
    g = torch.Generator().manual_seed(31 + D)
    lengths = torch.randint(1, T_cap - steps, (B,), generator=g).to(torch.int32)
    lengths[3] = 0                      # an empty sequence
    lengths[5] = T_cap - steps          # the longest one
    case = inputs.make_case(B, Hq, Hkv, D, T_cap, lengths + 1, "bf16", seed=77 + D)
    dev = torch.device("cuda")
    kc, vc = case.k_cache.to(dev, copy=True), case.v_cache.to(dev, copy=True)
    L = lengths.to(dev, copy=True)
    cache = kvd.KVCache(kc, vc, L, Hq)
    cache.set_variant(VARIANTS[variant])
    if splits:
        cache.set_num_splits(splits)
    k_ref, v_ref = inputs.host_array(case.k_cache), inputs.host_array(case.v_cache)
    L_ref = lengths.numpy().copy()
    try:
        for step in range(steps):
            gs = torch.Generator().manual_seed(1000 * step + D)
            kn = torch.randn(B, Hkv, D, generator=gs).to(torch.bfloat16)
            vn = torch.randn(B, Hkv, D, generator=gs).to(torch.bfloat16)
            q = torch.randn(B, Hq, D, generator=gs).to(torch.bfloat16)
            say(f"consecutive steps {variant} Hq={Hq} D={D} splits={splits}: step {step}")
            out = cache.step(kn.to(dev), vn.to(dev), q.to(dev), scale=D ** -0.5)
            k_ref, v_ref, L_ref, _ = oracle.append(k_ref, v_ref, L_ref, inputs.host_array(kn), inputs.host_array(vn))
            ref = oracle.decode_attention(inputs.host_array(q), k_ref, v_ref, L_ref, D ** -0.5, oracle.BF16)
            assert rel_err_rows(to_f64(out), ref) <= TOL_BF16, step
        assert cache.status() == kvd.KVD_OK
        torch.cuda.synchronize()
    finally:
        cache.close()
    assert np.array_equal(L.cpu().numpy(), L_ref)
    assert np.array_equal(inputs.host_array(kc), k_ref) and np.array_equal(inputs.host_array(vc), v_ref)


@pytest.mark.parametrize("variant", ["lds", "valu"])
def test_batch_past_the_sort_limit(variant):
    """2100 sequences (more than the combine's length sort takes, so every
    step dispatches in batch order) with ragged short lengths, over two
    consecutive steps on one handle; 2000 sequences (sorted dispatch from the
    second step on) alongside."""
    for B in (2100, 2000):
        g = torch.Generator().manual_seed(B)
        lengths = torch.randint(0, 62, (B,), generator=g).to(torch.int32)
        case = inputs.make_case(B, 8, 1, 64, 64, lengths + 1, "bf16", seed=B)
        dev = torch.device("cuda")
        kc, vc = case.k_cache.to(dev, copy=True), case.v_cache.to(dev, copy=True)
        L = lengths.to(dev, copy=True)
        cache = kvd.KVCache(kc, vc, L, 8)
        cache.set_variant(VARIANTS[variant])
        k_ref, v_ref, L_ref = inputs.host_array(case.k_cache), inputs.host_array(case.v_cache), lengths.numpy().copy()
        try:
            for step in range(2):
                gs = torch.Generator().manual_seed(7 * step + B)
                kn = torch.randn(B, 1, 64, generator=gs).to(torch.bfloat16)
                vn = torch.randn(B, 1, 64, generator=gs).to(torch.bfloat16)
                q = torch.randn(B, 8, 64, generator=gs).to(torch.bfloat16)
                say(f"batch {B} {variant}: step {step}")
                out = cache.step(kn.to(dev), vn.to(dev), q.to(dev), scale=0.125)
                k_ref, v_ref, L_ref, _ = oracle.append(k_ref, v_ref, L_ref, inputs.host_array(kn),
                                                       inputs.host_array(vn))
                ref = oracle.decode_attention(inputs.host_array(q), k_ref, v_ref, L_ref, 0.125, oracle.BF16)
                torch.cuda.synchronize()
                assert cache.status() == kvd.KVD_OK
                assert np.array_equal(L.cpu().numpy(), L_ref)
                assert np.array_equal(inputs.host_array(kc), k_ref)
                err = rel_err_rows(to_f64(out), ref)
                say(f"batch {B} {variant}: step {step} max row-relative error {err:.3e}")
                assert err <= TOL_BF16, err
        finally:
            cache.close()


def test_cache_past_4_gib():
    """An MHA cache of 5.4 GB per tensor (64 sequences, 40 KV heads, 8192
    tokens, d = 128): byte offsets of the later sequences pass 2^32.  One
    decode step at full length on the automatic plan; the first, a middle
    and the last sequence are checked against the oracle on their own
    slices (append bit for bit, attention to the bf16 tolerance)."""
    B, H, T, D = 64, 40, 8192, 128
    dev = torch.device("cuda")
    g = torch.Generator(device=dev).manual_seed(4321)
    kc = torch.randn(B, H, T, D, generator=g, device=dev).to(torch.bfloat16)
    vc = torch.randn(B, H, T, D, generator=g, device=dev).to(torch.bfloat16)
    assert kc.numel() * 2 > 2 ** 32
    lengths = torch.randint(T - 64, T, (B,), generator=g, device=dev).to(torch.int32)
    kn, vn = (torch.randn(B, H, D, generator=g, device=dev).to(torch.bfloat16) for _ in range(2))
    q = torch.randn(B, H, D, generator=g, device=dev).to(torch.bfloat16)
    picks = [0, B // 2, B - 1]
    before = {b: (inputs.host_array(kc[b:b + 1]), inputs.host_array(vc[b:b + 1])) for b in picks}
    L0 = lengths.cpu().numpy()
    cache = kvd.KVCache(kc, vc, lengths, H)
    try:
        say(f"cache past 4 GiB: B={B} H={H} T={T} D={D} plan={cache.plan()}")
        out = cache.step(kn, vn, q, scale=D ** -0.5)
        torch.cuda.synchronize()
        assert cache.status() == kvd.KVD_OK
    finally:
        cache.close()
    assert np.array_equal(lengths.cpu().numpy(), L0 + 1)
    for b in picks:
        k1, v1, L1, _ = oracle.append(*before[b], L0[b:b + 1], inputs.host_array(kn[b:b + 1]),
                                      inputs.host_array(vn[b:b + 1]))
        assert np.array_equal(inputs.host_array(kc[b:b + 1]), k1) and np.array_equal(inputs.host_array(vc[b:b + 1]), v1)
        ref = oracle.decode_attention(inputs.host_array(q[b:b + 1]), k1, v1, L1, D ** -0.5, oracle.BF16)
        err = rel_err_rows(to_f64(out[b:b + 1]), ref)
        say(f"cache past 4 GiB: sequence {b} max row-relative error {err:.3e}")
        assert err <= TOL_BF16, err
    del kc, vc, out, cache
    torch.cuda.empty_cache()  # return the 11 GB to the device for the tests after this one
