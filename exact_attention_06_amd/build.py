"""Build the HIP library ``libfa.so`` in-tree with hipcc for gfx950.

Usage: ``python -m exact_attention_06_amd.build`` (or ``build()`` from Python).
Every source in ``csrc/`` is compiled to an object under ``_build/`` (in
parallel), then linked into ``exact_attention_06_amd/libfa.so``.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")
ARCH = "gfx950"

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in the generated code.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the attention library)")


def _compile(src: str, obj: str) -> tuple[str, int, str]:
    cmd = [hipcc(), *COMMON_FLAGS, "-c", src, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (p.stdout + p.stderr).splitlines()
                     if "unknown target feature" not in line and line.strip())
    return src, p.returncode, out


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every csrc/*.hip and link libfa.so; returns the library path. Raises on failure."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    errors = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for src, rc, out in ex.map(lambda a: _compile(*a), zip(srcs, objs)):
            if out and (verbose or rc != 0):
                print(out, file=sys.stderr)
            if rc != 0:
                errors.append(src)
    if errors:
        raise RuntimeError(f"hipcc failed for: {', '.join(os.path.basename(e) for e in errors)}")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("link failed:\n" + p.stdout + p.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
