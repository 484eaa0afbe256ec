"""Build ``libkvdecode.so`` (the C-ABI library) for gfx950 with hipcc.

Every ``csrc/*.hip`` file is compiled to an object in ``_build/`` and the
objects are linked into ``multiquery_decode_attention_amd/libkvdecode.so``,
next to this file, so the library travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvdecode.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


# Per-file extra flags.  The LDS-staged kernels keep their matrix-core
# accumulators in ordinary VGPRs: its rare softmax rescale multiplies them on
# the vector ALU, and accumulators in AGPRs made the compiler copy all of
# them between register files on every loop iteration.
FILE_FLAGS = {
    "kvd_partial_lds.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "kvd_partial_lds_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "kvd_partial_wave_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "kvd_partial_xchg.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(extra=(), out: str = LIB, jobs: int = 8) -> str:
    """Compile and link the library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc link failed")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
