#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

A step is the whole hot path for one decode step of one attention layer:
append every sequence's new K/V token to its cache, then attend every query
head over its sequence's valid prefix (split-KV partial pass + log-sum-exp
combine), issued as one kvdecode_append_attend call.  Inputs are seeded
synthetic tensors resident in HBM before the timed region.  Several
independent cache copies are cycled so that no step finds its cache in the
256 MB last-level cache (as in a model whose other layers' caches are read in
between).

Each workload runs W warm-up steps, then K steps with nothing recorded on the
stream (the value pass), then K more steps with HIP events on the partial pass
and the combine, read after every step (the kernel-time pass).  The events
ride on the launches (the dispatch stamps each kernel's start and end), so
they add no command to the stream and time the kernels alone.

Prints one JSON line:
  value        value pass: step throughput in algorithmic GB/s (K/V of the
               valid prefixes + q + out + the appended token), whole job
  attend       kernel-time pass: median partial + combine time per step, and
               the algorithmic bytes of attention (K/V + q + out) over it, in
               GB/s and as a fraction of the 8 TB/s HBM peak
  roofline     the partial-pass kernel's algorithmic GB/s (K/V + q per launch
               / its mean launch time in the kernel-time pass) against the
               8 TB/s HBM peak
  cpu_baseline the fp64 CPU oracle on full steps of the same workload, on the
               host's cores
  extra        the same figures for every other workload, measured in this run
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "longctx_mqa_bf16"
MIN_ROTATION_BYTES = 2 << 30  # cycle >= 2 GiB of caches per round of steps
CPU_BASELINE_SECONDS = 10.0  # oracle time spent on the CPU baseline


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# Sources that define each partial-pass kernel (the roofline kernel).
KERNEL_SOURCES = {
    "lds": ["kvd_partial_lds.hip", "kvd_lds_common.h", "kvd_mfma_common.h", "kvd_internal.h"],
    "lds_fp8": ["kvd_partial_lds_fp8.hip", "kvd_fp8_common.h", "kvd_lds_common.h", "kvd_mfma_common.h",
                "kvd_internal.h"],
    "wave_fp8": ["kvd_partial_wave_fp8.hip", "kvd_fp8_common.h", "kvd_lds_common.h", "kvd_mfma_common.h",
                 "kvd_internal.h"],
    "xchg_fp8": ["kvd_partial_xchg.hip", "kvd_fp8_common.h", "kvd_lds_common.h", "kvd_mfma_common.h",
                 "kvd_internal.h"],
    "mfma": ["kvd_partial_mfma.hip", "kvd_mfma_common.h", "kvd_internal.h"],
    "valu": ["kvd_partial_valu.hip", "kvd_internal.h"],
}


def kernel_source_sha(variant: str = "lds") -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "multiquery_decode_attention_amd", "csrc")
    for name in KERNEL_SOURCES[variant]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def traffic_key(workload: str, page_size: int = 0, kv_dtype: str = "", new_tokens: int = 1) -> str:
    """Name of a workload's traffic record (and profile summaries)."""
    return (workload + (f"_paged{page_size}" if page_size else "") + (f"_{kv_dtype}" if kv_dtype else "")
            + (f"_tq{new_tokens}" if new_tokens > 1 else ""))


def measured_traffic(key: str, variant: str):
    """HBM bytes per partial-pass launch from committed rocprofv3 counter
    runs, or None when absent, taken on another kernel, or taken before the
    kernel's sources last changed."""
    path = os.path.join(ROOT, "profiles", f"traffic_{key}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel") != f"partial_{variant}_kernel" or \
            rec.get("kernel_source_sha") != kernel_source_sha(variant):
        return None
    return rec.get("hbm_bytes_per_launch")


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--splits", type=int, default=0, help="force split count (0 = plan)")
    ap.add_argument("--variant", default="auto", choices=["auto", "valu", "mfma", "lds", "wave", "xchg"])
    ap.add_argument("--cache-copies", type=int, default=0, help="0 = enough for 2 GiB")
    ap.add_argument("--page-size", type=int, default=0,
                    help="paged cache with this many tokens per page (0 = contiguous cache)")
    ap.add_argument("--kv-dtype", default="", choices=["", "fp8"],
                    help="fp8: the cache as E4M3 codes with per-row power-of-two scales "
                         "(bf16 queries and outputs); default: the workload's own dtype")
    ap.add_argument("--new-tokens", type=int, default=1,
                    help="tokens appended and attended per sequence per step (>1: a speculative-"
                         "verify step through kvdecode_append_attend_multi)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip measuring the other workloads (the 'extra' field)")
    ap.add_argument("--extra-steps", type=int, default=50, help="steps per pass for each other workload")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run plain device-to-device copies of MIB MiB (counter calibration)")
    return ap.parse_args(argv)


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import multiquery_decode_attention_amd as kvd
    from multiquery_decode_attention_amd import inputs, traffic

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    kvd.library()  # fail loudly before any work if the HIP library is missing
    if args.calibrate_copy:
        return calibrate_copy(args.calibrate_copy, args.steps)
    if args.new_tokens < 1 or args.new_tokens > kvd.KVD_MAX_NEW_TOKENS:
        print(f"--new-tokens must be 1..{kvd.KVD_MAX_NEW_TOKENS}", file=sys.stderr)
        sys.exit(2)
    w = inputs.WORKLOADS[args.workload]
    if args.kv_dtype == "fp8" and w.dtype != "bf16":
        print("--kv-dtype fp8 takes a bf16 workload", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(torch.device("cuda:0"))

    m = measure(w, args, args.steps, args.warmup, keep_first_copy=not args.no_cpu_baseline)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, m["first_copy"], w.T_cap, args.kv_dtype == "fp8", args.new_tokens)
    m.pop("first_copy", None)
    torch.cuda.empty_cache()

    extra = None
    if not args.no_extra:
        # the other workloads, each measured the same way in this run (fewer
        # steps), with the same cache type, layout and new-token count
        extra = {}
        for name, wx in inputs.WORKLOADS.items():
            if name == w.name or (args.kv_dtype == "fp8" and wx.dtype != "bf16"):
                continue
            ax = argparse.Namespace(**{**vars(args), "splits": 0, "variant": "auto", "cache_copies": 0})
            mx = measure(wx, ax, args.extra_steps, max(2, args.warmup // 2), keep_first_copy=False)
            extra[name] = {k: mx[k] for k in ("ms_per_step", "value", "tokens_per_s", "attend", "roofline",
                                               "plan")}
            extra[name]["roofline"] = {k: mx["roofline"][k] for k in ("bound", "achieved", "unit", "frac")}
            torch.cuda.empty_cache()

    fp8, tq = args.kv_dtype == "fp8", args.new_tokens
    plan = m["plan"]
    result = {
        "metric": "decode-attention KV-cache HBM GB/s (% of peak) and tokens/sec at 1 GPU",
        "value": m["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": ("synthetic (seeded random E4M3 cache codes and exponents, N(0,1) bf16 queries and new rows)"
                 if fp8 else "synthetic (seeded N(0,1) caches and queries)"),
        "pct_of_peak": round(m["value"] / traffic.MI355X_HBM_PEAK_GBPS, 4),
        "tokens_per_s": m["tokens_per_s"],
        "attend": m["attend"],
        "kernel_us": m["kernel_us"],
        "partial_tflops": m["partial_tflops"],
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "head_dim": w.D,
                   "T": w.T, "cache_dtype": "fp8_e4m3" if fp8 else w.dtype, "num_splits": plan["num_splits"],
                   "split_tokens": plan["split_tokens"], "variant": plan["variant"],
                   "cache_copies": m["copies"], "seed": w.seed, "page_size": args.page_size or None,
                   "new_tokens": tq},
        "roofline": m["roofline"],
        "cpu_baseline": cpu,
        "extra": extra,
        "device": device_info(),
    }
    print(json.dumps(result), flush=True)


def measure(w, args, K, W, keep_first_copy=False) -> dict:
    """One workload: build cache copies, run W warm-up steps, K timed steps
    with nothing recorded on the stream (the `value` pass), then K more steps
    with HIP events on the partial pass and the combine, read after every
    step (the kernel-time pass).  Returns the figures of both passes."""
    import statistics
    import torch
    import multiquery_decode_attention_amd as kvd
    from multiquery_decode_attention_amd import inputs, traffic

    dev = torch.device("cuda:0")
    fp8 = args.kv_dtype == "fp8"
    tq = args.new_tokens
    kv_bytes_one = (traffic.kv_read_bytes_fp8(w.Hkv, w.D, [w.T_cap] * w.B) if fp8 else
                    traffic.kv_read_bytes(w.Hkv, w.D, w.elem_bytes, [w.T_cap] * w.B))
    n_steps = W + 2 * K
    R = args.cache_copies or max(1, math.ceil(MIN_ROTATION_BYTES / kv_bytes_one))
    R = min(R, n_steps)
    appends_per_copy = math.ceil(n_steps / R)
    # Each copy starts appends_per_copy tokens short of the workload's lengths
    # so that its last step attends exactly them: the cache capacity is the
    # workload's own, and attended lengths stay within appends_per_copy of it.
    T_cap = w.T_cap
    final = inputs.attended_lengths(w)
    attended = (final - tq * (appends_per_copy - 1)).clamp(min=tq)  # after the first append
    log(f"workload {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} T={w.T} dtype={w.dtype}; "
        f"{R} cache copies of {kv_bytes_one / 1e6:.0f} MB, capacity {T_cap}")

    variant = {"auto": kvd.KVD_VARIANT_AUTO, "valu": kvd.KVD_VARIANT_VALU,
               "mfma": kvd.KVD_VARIANT_MFMA, "lds": kvd.KVD_VARIANT_LDS,
               "wave": kvd.KVD_VARIANT_WAVE, "xchg": kvd.KVD_VARIANT_XCHG}[args.variant]
    copies = []
    for r in range(R):
        keep = {}
        if fp8:
            case = inputs.make_fp8_case(w.B, w.Hq, w.Hkv, w.D, T_cap, attended, seed=w.seed + 1000 * r,
                                        device=dev, new_tokens=tq if tq > 1 else None)
            if args.page_size:
                # codes and exponents in shuffled pages under one block table
                bt, num_pages = inputs.paged_layout(w.B, T_cap, args.page_size, seed=w.seed + 1000 * r + 1)
                keep = {n: inputs.to_pages(x, bt, args.page_size, num_pages)
                        for n, x in (("kc", case.k_codes), ("ke", case.k_exp), ("vc", case.v_codes),
                                     ("ve", case.v_exp))}
                keep["block_table"] = bt.to(dev)
                cache = kvd.KVCache(keep["kc"], keep["vc"], case.lengths0, w.Hq, block_table=keep["block_table"],
                                    k_exp=keep["ke"], v_exp=keep["ve"])
            else:
                cache = kvd.KVCache(case.k_codes, case.v_codes, case.lengths0, w.Hq, k_exp=case.k_exp,
                                    v_exp=case.v_exp)
        else:
            if tq > 1:
                case = inputs.make_multi_case(w.B, w.Hq, w.Hkv, w.D, T_cap, attended - tq, tq, w.dtype,
                                              seed=w.seed + 1000 * r, device=dev)
            else:
                case = inputs.make_case(w.B, w.Hq, w.Hkv, w.D, T_cap, attended, w.dtype,
                                        seed=w.seed + 1000 * r, device=dev, k_scale=w.k_scale)
            if args.page_size:
                # the same caches laid out in shuffled pages; the page pools and
                # block table replace the contiguous tensors on the device
                kp, vp, bt = inputs.make_paged(case.k_cache, case.v_cache, args.page_size,
                                               seed=w.seed + 1000 * r + 1)
                keep = {"k_pages": kp, "v_pages": vp, "block_table": bt.to(dev)}
                cache = kvd.KVCache(kp, vp, case.lengths0, w.Hq, block_table=keep["block_table"])
            else:
                cache = kvd.KVCache(case.k_cache, case.v_cache, case.lengths0, w.Hq)
        cache.set_variant(variant)
        cache.set_num_splits(args.splits)
        cache.reserve(tq)  # device workspace allocated now, not inside the timed steps
        copies.append({"case": case, "cache": cache, "out": torch.empty_like(case.q),
                       "len": case.lengths0.cpu().tolist(), "keep": keep})
    plan = copies[0]["cache"].plan(tq)  # the plan of a step with tq new tokens
    log(f"plan {plan}")
    torch.cuda.synchronize()

    # The timed loops call the C ABI directly with arguments marshalled once
    # (shapes were checked when the copies were built).
    lib = kvd.library()
    stream = torch.cuda.current_stream().cuda_stream
    for c in copies:
        cs = c["case"]
        c["args"] = (c["cache"].handle, cs.k_new.data_ptr(), cs.v_new.data_ptr(), cs.q.data_ptr(),
                     c["out"].data_ptr(), float(cs.scale), stream)

    def step(i):
        if tq > 1:  # append tq drafted tokens, then attend their queries causally
            a = copies[i % R]["args"]
            rc = lib.kvdecode_append_attend_multi(a[0], tq, *a[1:])
        else:
            rc = lib.kvdecode_append_attend(*copies[i % R]["args"])  # append, then attend
        if rc:
            raise kvd.KvdError(rc, "decode step")

    # Byte and FLOP counts of every step, from the lengths it attends (every
    # step appends tq tokens to each sequence of its copy); computed before
    # the timed loops so that they only issue the steps.
    lens = [list(c["len"]) for c in copies]
    step_bytes, partial_bytes, flops = [], [], []
    for i in range(n_steps):
        L = lens[i % R] = [n + tq for n in lens[i % R]]
        if tq > 1:
            # the cache is read once for all tq queries; q, out and the
            # appended rows scale with tq (q and out stay bf16 over fp8)
            if fp8:
                kv, app = traffic.kv_read_bytes_fp8(w.Hkv, w.D, L), traffic.append_bytes_fp8(w.B, w.Hkv, w.D)
            else:
                kv = traffic.kv_read_bytes(w.Hkv, w.D, w.elem_bytes, L)
                app = traffic.append_bytes(w.B, w.Hkv, w.D, w.elem_bytes)
            step_bytes.append(kv + 2 * w.B * w.Hq * tq * w.D * w.elem_bytes + app * tq)
            partial_bytes.append(kv + w.B * w.Hq * tq * w.D * w.elem_bytes)
        elif fp8:
            step_bytes.append(traffic.attend_bytes_fp8(w.B, w.Hq, w.Hkv, w.D, L) +
                              traffic.append_bytes_fp8(w.B, w.Hkv, w.D))
            partial_bytes.append(traffic.partial_pass_bytes_fp8(w.B, w.Hq, w.Hkv, w.D, L))
        else:
            step_bytes.append(traffic.attend_bytes(w.B, w.Hq, w.Hkv, w.D, w.elem_bytes, L) +
                              traffic.append_bytes(w.B, w.Hkv, w.D, w.elem_bytes))
            partial_bytes.append(traffic.partial_pass_bytes(w.B, w.Hq, w.Hkv, w.D, w.elem_bytes, L))
        flops.append(traffic.attend_flops(w.Hq * tq, w.D, L))
    for c, L in zip(copies, lens):
        c["len"] = L  # the lengths each copy holds once every step has run

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    for c in copies:
        assert c["cache"].status() == kvd.KVD_OK
    torch.cuda.synchronize()

    # value pass: K steps, nothing recorded on the stream
    t0 = time.perf_counter()
    for i in range(W, W + K):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # kernel-time pass: K more steps whose partial and combine launches carry
    # HIP events, read at once (per-step kernel durations)
    for c in copies:
        kvd.kvdecode_timing_enable(c["cache"].handle, 1, kvd.KVD_TIME_PARTIAL | kvd.KVD_TIME_COMBINE)
    part_us, comb_us = [], []
    for i in range(W + K, W + 2 * K):
        step(i)
        t = kvd.kvdecode_timing_read(copies[i % R]["cache"].handle)
        assert t["n_attend"] == 1, t
        part_us.append(t["partial_ms"] * 1e3)
        comb_us.append(t["combine_ms"] * 1e3)
    torch.cuda.synchronize()
    for c in copies:
        kvd.kvdecode_timing_enable(c["cache"].handle, 0, 0)
        assert c["cache"].status() == kvd.KVD_OK

    value = sum(step_bytes[W:W + K]) / elapsed / 1e9
    ms_per_step = elapsed * 1e3 / K
    kb = partial_bytes[W + K:]
    attend_us = [p + c for p, c in zip(part_us, comb_us)]
    partial_mean_us = statistics.fmean(part_us)
    achieved = statistics.fmean(kb) / (partial_mean_us * 1e-6) / 1e9
    tflops = statistics.fmean(flops[W + K:]) / (partial_mean_us * 1e-6) / 1e12
    # attend: bytes the step must move (K/V + q + out) over partial + combine
    attend_bytes = [sb - (traffic.append_bytes_fp8(w.B, w.Hkv, w.D) if fp8 else
                          traffic.append_bytes(w.B, w.Hkv, w.D, w.elem_bytes)) * tq for sb in step_bytes[W + K:]]
    attend_gbps = statistics.median(b / (t * 1e-6) / 1e9 for b, t in zip(attend_bytes, attend_us))
    attend_med = statistics.median(attend_us)
    log(f"step {ms_per_step * 1e3:.1f} us; partial {partial_mean_us:.1f} us (median "
        f"{statistics.median(part_us):.1f}); attend median {attend_med:.1f} us, {attend_gbps:.0f} GB/s "
        f"({attend_gbps / traffic.MI355X_HBM_PEAK_GBPS:.1%} of peak)")

    # kernel name suffix of the fp8 kernels
    kvariant = plan["variant"] + ("_fp8" if fp8 else "")
    # The partial pass is HBM-bound unless its arithmetic intensity passes
    # the bf16 matrix-core ridge (peak FLOP/s over peak bytes/s, about 312
    # FLOP/B): with many query rows per KV head (48 heads times several new
    # tokens) it is a contraction and is measured against the matrix peak.
    intensity = sum(flops) / sum(partial_bytes)
    ridge = traffic.MI355X_BF16_DENSE_TFLOPS * 1e12 / (traffic.MI355X_HBM_PEAK_GBPS * 1e9)
    traffic_rec = measured_traffic(traffic_key(w.name, args.page_size, args.kv_dtype, tq), kvariant)
    if w.dtype == "bf16" and intensity > ridge:
        roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": traffic.MI355X_BF16_DENSE_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tflops / traffic.MI355X_BF16_DENSE_TFLOPS, 4)}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": traffic.MI355X_HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(achieved / traffic.MI355X_HBM_PEAK_GBPS, 4)}
    roofline.update({"traffic": traffic_rec, "kernel": f"partial_{kvariant}_kernel",
                     "intensity_flop_per_byte": round(intensity, 1)})
    out = {
        "value": round(value, 2),
        "ms_per_step": round(ms_per_step, 5),
        "tokens_per_s": round(w.B * tq * K / elapsed, 1),
        "attend": {"us_median": round(attend_med, 2),
                   "partial_us_median": round(statistics.median(part_us), 2),
                   "combine_us_median": round(statistics.median(comb_us), 2),
                   "GBps": round(attend_gbps, 1),
                   "frac": round(attend_gbps / traffic.MI355X_HBM_PEAK_GBPS, 4),
                   "tokens_per_s": round(w.B * tq / (attend_med * 1e-6), 1), "steps": K},
        "kernel_us": {"partial_mean": round(partial_mean_us, 2), "combine_mean": round(statistics.fmean(comb_us), 2)},
        "partial_tflops": round(tflops, 2),
        "roofline": roofline,
        "plan": plan,
        "copies": R,
    }
    if keep_first_copy:
        out["first_copy"] = copies[0]
    for c in copies:
        c["cache"].close()
    return out


def device_info() -> dict:
    """The GPU the run used, as the runtime reports it (peak figures are
    MI355X's: an arch other than gfx950 makes them meaningless)."""
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2 ** 30, 1)}


def calibrate_copy(mib: int, reps: int):
    """Plain device-to-device copies of a known size: the per-dispatch
    FETCH_SIZE / WRITE_SIZE counters of these copies convert the counters of
    the attention kernels into bytes."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / reps
    print(json.dumps({"calibrate_copy_bytes": n, "reps": reps,
                      "copy_GBps_read_plus_write": round(2 * n / sec / 1e9, 1)}), flush=True)


def cpu_baseline(w, copy, T_cap, fp8=False, tq=1):
    """The fp64 oracle (test infrastructure) on whole steps of the same
    workload: the first copy's cache as it now stands, attended again and
    again until about CPU_BASELINE_SECONDS have run (at least once)."""
    import numpy as np
    import oracle
    from multiquery_decode_attention_amd import inputs, traffic

    case = copy["case"]
    L = np.asarray(copy["len"], dtype=np.int32)
    threads = oracle.default_threads()
    log(f"cpu baseline: copying {w.name} cache to host, oracle on {threads} threads "
        f"({os.cpu_count()} CPUs on the host, {len(os.sched_getaffinity(0))} in this process's affinity)")
    if fp8:
        host = [t.cpu().numpy() for t in (case.k_codes, case.k_exp, case.v_codes, case.v_exp)]
        q = case.q.float().cpu().numpy()
        def run():
            if tq > 1:
                oracle.decode_attention_fp8_multi(q, *host, L, np.full(w.B, tq), case.scale, threads=threads)
            else:
                oracle.decode_attention_fp8(q, *host, L, case.scale, threads=threads)
        b = traffic.kv_read_bytes_fp8(w.Hkv, w.D, L.tolist()) + 2 * w.B * w.Hq * tq * w.D * 2
    else:
        k = inputs.host_array(case.k_cache)
        v = inputs.host_array(case.v_cache)
        q = inputs.host_array(case.q)
        dt = oracle.BF16 if w.dtype == "bf16" else oracle.F32
        def run():
            if tq > 1:
                oracle.decode_attention_multi(q, k, v, L, np.full(w.B, tq), case.scale, dt, threads=threads)
            else:
                oracle.decode_attention(q, k, v, L, case.scale, dt, threads=threads)
        b = traffic.attend_bytes(w.B, w.Hq * tq, w.Hkv, w.D, w.elem_bytes, L.tolist())
    # whole attend steps, repeated until about CPU_BASELINE_SECONDS have run
    runs, t0 = 0, time.perf_counter()
    while runs == 0 or time.perf_counter() - t0 < CPU_BASELINE_SECONDS:
        run()
        runs += 1
    total = time.perf_counter() - t0
    sec = total / runs
    log(f"cpu baseline: {runs} steps in {total:.1f} s, {sec:.2f} s per step")
    return {"value": round(b / sec / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{runs} full attend steps of {w.name} (B={w.B}, all {w.Hq} heads, "
                      f"{int(L.sum())} cached tokens in all), fp64, {total:.1f} s in all, {sec:.2f} s per step",
            "tokens_per_s": round(w.B * tq / sec, 2),
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
