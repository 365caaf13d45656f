"""MFMA data hazards in the built kernels (CPU only: hipcc cross-compiles).

The NT kernels write their MFMAs as inline assembly, so the wait states
around them are placed by hand and the compiler's own hazard recognizer does
not check them.  These tests compile every kernel-instance unit to gfx950
assembly with the library's own flags and run the static check of
tests/mfma_hazards.py over every kernel; a small snippet with planted
hazards (and a corrected copy of it) shows that the check finds each kind.
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import mfma_hazards  # noqa: E402

from software_pipelined_tiled_pipeline_amd import build  # noqa: E402

UNITS = [u for u in build.UNITS if u.startswith("inst_")]


def hipcc_available():
    return shutil.which(build.hipcc()) or os.path.exists(build.hipcc())


def device_asm(src_path, out_path):
    cmd = [build.hipcc(), *build.HIPCC_FLAGS, "-S", "--cuda-device-only", src_path, "-o", out_path]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    with open(out_path) as f:
        return f.read()


@pytest.fixture(scope="module")
def unit_asm():
    if not hipcc_available():
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as tmp:
        def one(u):
            return u, device_asm(os.path.join(build.CSRC, u), os.path.join(tmp, u + ".s"))
        with ThreadPoolExecutor(len(UNITS)) as pool:
            return dict(pool.map(one, UNITS))


@pytest.mark.parametrize("unit", UNITS)
def test_no_mfma_hazards_in_kernels(unit_asm, unit):
    asm = unit_asm[unit]
    funcs = mfma_hazards.parse_functions(asm)
    kernels = [n for n in funcs if "nt_swap_kernel" in n or "nt_ws_kernel" in n or "nt_ws_persistent" in n]
    # both variants, four stage counts, two tile sizes, with and without a K
    # split on the small tile (and the persistent schedule with the direct loader)
    assert len(kernels) == (32 if unit.endswith("direct.hip") else 24), len(kernels)
    hazards, mfmas = mfma_hazards.check_asm(asm)
    assert mfmas > 1000
    assert not hazards, "\n".join(f"{h.kind} line {h.line}: {h.text} ({h.detail})" for h in hazards[:20])


PLANTED = r"""
#include <hip/hip_runtime.h>
// Each kernel issues one hand-written sequence; `fixed` selects the copy
// with the wait states / counter wait in place.
template <int KIND, bool FIXED>
__global__ void planted(float *out) {
  if constexpr (KIND == 0) {  // VALU write of a source, MFMA right after
    if constexpr (FIXED)
      asm volatile("v_mov_b32 v8, 0\n\ts_nop 1\n\tv_mfma_f32_16x16x32_f16 a[0:3], v[8:11], v[12:15], a[0:3]"
                   ::: "v8", "v9", "v10", "v11", "v12", "v13", "v14", "v15", "a0", "a1", "a2", "a3");
    else
      asm volatile("v_mov_b32 v8, 0\n\tv_mfma_f32_16x16x32_f16 a[0:3], v[8:11], v[12:15], a[0:3]"
                   ::: "v8", "v9", "v10", "v11", "v12", "v13", "v14", "v15", "a0", "a1", "a2", "a3");
  } else if constexpr (KIND == 1) {  // MFMA result read by a VALU too soon
    if constexpr (FIXED)
      asm volatile("v_mfma_f32_16x16x32_f16 a[0:3], v[8:11], v[12:15], a[0:3]\n\ts_nop 7\n\ts_nop 7\n\t"
                   "v_accvgpr_read_b32 v0, a0"
                   ::: "v0", "v8", "v9", "v10", "v11", "v12", "v13", "v14", "v15", "a0", "a1", "a2", "a3");
    else
      asm volatile("v_mfma_f32_16x16x32_f16 a[0:3], v[8:11], v[12:15], a[0:3]\n\ts_nop 3\n\t"
                   "v_accvgpr_read_b32 v0, a0"
                   ::: "v0", "v8", "v9", "v10", "v11", "v12", "v13", "v14", "v15", "a0", "a1", "a2", "a3");
  } else {  // LDS load of a source, MFMA before the counter wait
    if constexpr (FIXED)
      asm volatile("ds_read_b128 v[8:11], v1\n\ts_waitcnt lgkmcnt(0)\n\t"
                   "v_mfma_f32_16x16x32_f16 a[0:3], v[8:11], v[12:15], a[0:3]"
                   ::: "v8", "v9", "v10", "v11", "v12", "v13", "v14", "v15", "a0", "a1", "a2", "a3");
    else
      asm volatile("ds_read_b128 v[8:11], v1\n\ts_nop 7\n\tv_mfma_f32_16x16x32_f16 a[0:3], v[8:11], v[12:15], a[0:3]"
                   ::: "v8", "v9", "v10", "v11", "v12", "v13", "v14", "v15", "a0", "a1", "a2", "a3");
  }
  out[threadIdx.x] = 0.0f;
}
template __global__ void planted<0, false>(float *);
template __global__ void planted<0, true>(float *);
template __global__ void planted<1, false>(float *);
template __global__ void planted<1, true>(float *);
template __global__ void planted<2, false>(float *);
template __global__ void planted<2, true>(float *);
"""


def test_planted_hazards_are_found():
    if not hipcc_available():
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "planted.hip")
        with open(src, "w") as f:
            f.write(PLANTED)
        asm = device_asm(src, os.path.join(tmp, "planted.s"))
    funcs = mfma_hazards.parse_functions(asm)
    expect = {0: "VALU_TO_MFMA", 1: "MFMA_RESULT", 2: "LOAD_TO_MFMA"}
    seen = 0
    for name, body in funcs.items():
        if "planted" not in name:
            continue
        kind = int(name.split("ILi")[1][0])
        fixed = name.split("ELb")[1][0] == "1"
        hazards = mfma_hazards.check_function(name, body)
        kinds = {h.kind for h in hazards}
        if fixed:
            assert not hazards, f"{name}: {hazards}"
        else:
            assert kinds == {expect[kind]}, f"{name}: {kinds}"
        seen += 1
    assert seen == 6
