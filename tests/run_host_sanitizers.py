"""Run the CPU test suite with the oracle and the library's host code
built under AddressSanitizer and UndefinedBehaviorSanitizer.

CPU only.  The oracle (oracle.c) is compiled with clang and both
sanitizers; the library is compiled as usual except that its host pass gets
the sanitizer flags (each through -Xarch_host, so no device code is
instrumented).  Both land in a temporary directory and are loaded in place
of the usual builds (KVD_ORACLE_LIBRARY, KVD_LIBRARY) by a pytest run of the
tests not marked gpu, with clang's sanitizer runtime preloaded into the
interpreter.  Leak checking is off: the interpreter and torch keep memory
until exit by design.  Any sanitizer report fails the run.

    python tests/run_host_sanitizers.py [extra pytest arguments]
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from multiquery_decode_attention_amd import _build  # noqa: E402

LLVM = "/opt/rocm/llvm"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def runtime() -> str:
    found = sorted(glob.glob(os.path.join(LLVM, "lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")))
    if not found:
        raise SystemExit("clang's AddressSanitizer runtime is not installed")
    return found[-1]


def main(argv) -> int:
    tmp = tempfile.mkdtemp(prefix="kvd_san_")
    oracle_so = os.path.join(tmp, "liboracle.so")
    subprocess.run([os.path.join(LLVM, "bin/clang"), "-O1", "-g", *SAN, "-std=c11", "-shared", "-fPIC", "-pthread",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", oracle_so, "-lm"], check=True)
    _build.BUILD = os.path.join(tmp, "objs")
    host_flags = ["-g"]
    for f in SAN:
        host_flags += ["-Xarch_host", f]
    lib_so = _build.build(extra=host_flags, out=os.path.join(tmp, "libkvdecode.so"))
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "KVD_LIBRARY": lib_so,
        "KVD_ORACLE_LIBRARY": oracle_so,
    })
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-q", "-x", *argv]
    print("sanitized libraries in", tmp, flush=True)
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
