"""Host-side checks of bench.py: the one-GPU guard, the kernel-source
hashes that tie counter records to the sources they were taken on, and the
traffic lookup that reports null for a record taken on other sources."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("gpus", [2, 8])
def test_more_than_one_gpu_is_refused(gpus):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(gpus)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_every_kernel_source_exists_and_hashes():
    csrc = os.path.join(ROOT, "multiquery_decode_attention_amd", "csrc")
    for variant, files in bench.KERNEL_SOURCES.items():
        for name in files:
            assert os.path.isfile(os.path.join(csrc, name)), (variant, name)
        sha = bench.kernel_source_sha(variant)
        assert len(sha) == 16 and int(sha, 16) >= 0


def test_traffic_record_only_for_its_kernel_and_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    sha = bench.kernel_source_sha("lds")
    rec = {"kernel": "partial_lds_kernel", "kernel_source_sha": sha, "hbm_bytes_per_launch": 12345}
    (prof / "traffic_w.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # the hashes read the sources under ROOT: keep the repository's
    monkeypatch.setattr(bench, "kernel_source_sha", lambda v: sha if v == "lds" else "0" * 16)
    assert bench.measured_traffic("w", "lds") == 12345
    assert bench.measured_traffic("w", "xchg_fp8") is None    # another kernel
    assert bench.measured_traffic("absent", "lds") is None
    rec["kernel_source_sha"] = "f" * 16                        # taken on older sources
    (prof / "traffic_w.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("w", "lds") is None


def test_traffic_keys():
    assert bench.traffic_key("longctx_mqa_bf16") == "longctx_mqa_bf16"
    assert bench.traffic_key("ragged_gqa_bf16", 256) == "ragged_gqa_bf16_paged256"
    assert bench.traffic_key("palm_mqa_bf16", 0, "fp8", 4) == "palm_mqa_bf16_fp8_tq4"


def test_cpu_baseline_repeats_whole_steps(monkeypatch):
    """The oracle baseline on the tiny workload's shape, on host tensors:
    whole steps repeated until the time budget has run, rates consistent
    with the step count."""
    import torch
    from multiquery_decode_attention_amd import inputs
    w = inputs.WORKLOADS["tiny_mqa_f32"]
    case = inputs.make_workload_case(w, device="cpu")
    copy = {"case": case, "len": (case.lengths0 + 1).tolist()}
    monkeypatch.setattr(bench, "CPU_BASELINE_SECONDS", 0.3)
    r = bench.cpu_baseline(w, copy, w.T_cap)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["cores"] >= 1 and r["value"] > 0
    runs = int(r["sample"].split()[0])
    assert runs >= 1 and "full attend steps of tiny_mqa_f32" in r["sample"]
    assert r["tokens_per_s"] > 0 and isinstance(case.q, torch.Tensor)
