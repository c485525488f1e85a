"""Builds libtwell.so (every HIP source under csrc/) for gfx950 with hipcc.

Each source is compiled to its own object in parallel, then the objects are
linked into one shared library.
"""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libtwell.so")
OBJ = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions: the compiler must not emit v_pk_* f32 math
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _filter(stderr: str) -> list[str]:
    return [ln for ln in stderr.splitlines() if "packed-fp32-ops" not in ln]


def _compile(src: str) -> tuple[str, int, list[str]]:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return obj, r.returncode, _filter(r.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source and link one shared library (always recompiles)."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = max(1, min(len(sources()), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(jobs) as ex:
        res = list(ex.map(_compile, sources()))
    errs = [ln for _, rc, e in res for ln in e]
    if any(rc != 0 for _, rc, _ in res):
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                        *[o for o, _, _ in res], "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc link failed:\n" + "\n".join(_filter(r.stderr)))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
