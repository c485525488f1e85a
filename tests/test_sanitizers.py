"""The C-ABI's host code and the oracle under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

- Every HIP source is compiled as for the library, with the sanitizers on the
  host pass only, and linked with ``tests/sanitize/abi_check.cpp``, which
  drives every entry point's argument checks and every workspace sizer over
  the edges of its arguments' ranges. No call it makes passes the checks, so
  nothing is launched and no GPU is needed.
- The oracle's C source is built with gcc and the same sanitizers, and
  ``tests/sanitize/oracle_run.py`` runs each of its functions on small inputs
  with AddressSanitizer preloaded.
Any sanitizer report aborts the run (no recovery), which fails the test."""
import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "activation_sparse_ffn_gemm_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}
# sanitizers on the host pass only; the sources are built without device code
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    return r


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    flags = ["--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, *flags, "-c", src, "-o", obj])
        return obj

    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "abi_check.o")
    _run([HIPCC, "-std=c++17", "-O1", "-g", *HOST_SAN, "-I", os.path.join(ROOT, "include"),
          "-c", os.path.join(SAN, "abi_check.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_check")
    _run([HIPCC, "--offload-arch=gfx950", *HOST_SAN, drv, *objs, "-o", exe])
    r = _run([exe], env={**os.environ, **SAN_ENV}, timeout=300)
    assert "abi_check ok" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libtwell_oracle_san.so")
    _run(["gcc", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-o", lib, os.path.join(ROOT, "oracle", "twell_oracle.c")])
    asan = _run(["gcc", "-print-file-name=libasan.so"]).stdout.strip()
    assert os.path.isabs(asan), "gcc has no AddressSanitizer runtime"
    env = {**os.environ, **SAN_ENV, "LD_PRELOAD": asan}
    r = _run([sys.executable, os.path.join(SAN, "oracle_run.py"), lib], env=env, timeout=600)
    assert "oracle_run ok" in r.stdout
