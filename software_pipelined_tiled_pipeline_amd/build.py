"""Builds libpgemm.so (HIP, gfx950 only) in-tree with hipcc.

The library is five translation units: the C ABI (argument checks,
planning, the int32 kernel) and four units of NT kernel instances (f16 and
bf16, each with the direct-to-LDS and the register-staged loader).  They are
compiled in parallel and linked into one shared library.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
UNITS = ["pgemm_api.hip", "inst_f16_direct.hip", "inst_f16_staged.hip", "inst_bf16_direct.hip",
         "inst_bf16_staged.hip"]
LIB = os.path.join(HERE, "libpgemm.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
_NOISE = "packed-fp32-ops"


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if _NOISE not in l and l.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed: " + " ".join(cmd) + "\n" + "\n".join(msgs))
    return msgs


def build(verbose: bool = False, lib: str = LIB, extra_flags=(), jobs: int = 0) -> str:
    """Compiles every unit (in parallel) and links libpgemm.so."""
    jobs = jobs or min(len(UNITS), os.cpu_count() or 1)
    with tempfile.TemporaryDirectory(prefix="pgemm_build_") as tmp:
        objs = [os.path.join(tmp, u.replace(".hip", ".o")) for u in UNITS]

        def compile_one(i):
            return _run([hipcc(), *HIPCC_FLAGS, *extra_flags, "-c", os.path.join(CSRC, UNITS[i]), "-o", objs[i]])

        with ThreadPoolExecutor(jobs) as pool:
            msgs = [m for ms in pool.map(compile_one, range(len(UNITS))) for m in ms]
        out = lib + ".tmp"
        msgs += _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out])
        if verbose and msgs:
            print("\n".join(msgs), file=sys.stderr)
        os.replace(out, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
