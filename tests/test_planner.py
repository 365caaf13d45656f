"""The host pipeline planner (stage/order validity, version counts, LDS
arena packing) through the C ABI, on the CPU.

Pins: the buffer-version model outputs printed by TileLang ch.22
("pipeline-sync-multibuffer") §3.4 for a 128x128x64 fp16 GEMM
(tests/golden/tilelang_buffer_model.txt); the version rule and its worked
cases in §2.4 (written in stage 0 and read in stage 2: three versions; read
in the stage that writes it: one; never written in the body: one; the
count drops by one when no writer precedes a reader in both order and
stage); the upstream stage vector quoted in §7.3 for the copy/copy/gemm
body at num_stages = 3 ([0, 0, 2]); the validity rules of §2.2.
"""
import ctypes
import os

import pytest

from software_pipelined_tiled_pipeline_amd import pgemm

HERE = os.path.dirname(os.path.abspath(__file__))
OK, ERR_NULL, ERR_SHAPE, ERR_STAGES = 0, 1, 2, 3
KIB = 1024


class Access(ctypes.Structure):
    _fields_ = [("stmt", ctypes.c_int32), ("buffer", ctypes.c_int32), ("write", ctypes.c_int32)]


class Block(ctypes.Structure):
    _fields_ = [("bytes", ctypes.c_int64), ("versions", ctypes.c_int32), ("align", ctypes.c_int32),
                ("start", ctypes.c_int32), ("end", ctypes.c_int32)]


@pytest.fixture(scope="module")
def L():
    L = pgemm.lib()
    I32P, I64P = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    L.pgemm_plan_versions.argtypes = [ctypes.c_int32, I32P, I32P, ctypes.c_int32, ctypes.POINTER(Access),
                                      ctypes.c_int32, I32P]
    L.pgemm_plan_versions.restype = ctypes.c_int
    L.pgemm_plan_arena.argtypes = [ctypes.c_int32, ctypes.POINTER(Block), I64P, I64P, I64P]
    L.pgemm_plan_arena.restype = ctypes.c_int
    return L


def versions(L, stage, order, accesses, n_buffers):
    n = len(stage)
    st = (ctypes.c_int32 * max(n, 1))(*stage)
    od = (ctypes.c_int32 * max(n, 1))(*order)
    acc = (Access * max(len(accesses), 1))(*[Access(*a) for a in accesses])
    out = (ctypes.c_int32 * max(n_buffers, 1))()
    status = L.pgemm_plan_versions(n, st, od, len(accesses), acc, n_buffers, out)
    return status, list(out)[:n_buffers]


def arena(L, blocks):
    arr = (Block * max(len(blocks), 1))(*[Block(*b) for b in blocks])
    offs = (ctypes.c_int64 * max(len(blocks), 1))()
    a, s = ctypes.c_int64(), ctypes.c_int64()
    status = L.pgemm_plan_arena(len(blocks), arr, offs, ctypes.byref(a), ctypes.byref(s))
    assert status == OK
    return a.value, s.value, list(offs)[:len(blocks)]


# ------------------------------------------------------------ versions

def test_versions_worked_cases(L):
    W, R = 1, 0
    # copy A (stage 0), copy B (stage 0), gemm reading both (stage 2): the
    # upstream stage vector [0, 0, 2] of the num_stages = 3 body
    assert versions(L, [0, 0, 2], [0, 1, 2], [(0, 0, W), (1, 1, W), (2, 0, R), (2, 1, R)], 2) == (OK, [3, 3])
    # num_stages = 2: consumer in stage 1 -> two versions
    assert versions(L, [0, 0, 1], [0, 1, 2], [(0, 0, W), (1, 1, W), (2, 0, R), (2, 1, R)], 2) == (OK, [2, 2])
    # written and read in the same stage, writer first: one version
    assert versions(L, [0, 0], [0, 1], [(0, 0, W), (1, 0, R)], 1) == (OK, [1])
    # never written in the body (an accumulator allocated outside): one
    assert versions(L, [0, 1], [0, 1], [(0, 0, R), (1, 0, R)], 1) == (OK, [1])
    # written in stage 0, read in stage 1 but before the writer in order:
    # use - def + 1 = 2 is tightened to 1
    assert versions(L, [0, 1], [1, 0], [(0, 0, W), (1, 0, R)], 1) == (OK, [1])
    # the same with the writer first in order keeps both versions
    assert versions(L, [0, 1], [0, 1], [(0, 0, W), (1, 0, R)], 1) == (OK, [2])
    # the kernels' own two-statement body: fill (stage 0) and MMA (stage S-1)
    for S in (1, 2, 3, 4):
        assert versions(L, [0, S - 1], [0, 1], [(0, 0, W), (1, 0, R)], 1) == (OK, [S])


def test_invalid_annotations(L):
    W, R = 1, 0
    # two statements with the same order
    assert versions(L, [0, 1], [0, 0], [(0, 0, W), (1, 0, R)], 1)[0] == ERR_STAGES
    # a reader in an earlier stage than its writer
    assert versions(L, [1, 0], [0, 1], [(0, 0, W), (1, 0, R)], 1)[0] == ERR_STAGES
    # same stage, reader ordered before the writer
    assert versions(L, [0, 0], [1, 0], [(0, 0, W), (1, 0, R)], 1)[0] == ERR_STAGES
    # negative stage, indices out of range
    assert versions(L, [-1, 0], [0, 1], [(0, 0, W), (1, 0, R)], 1)[0] == ERR_STAGES
    assert versions(L, [0, 1], [0, 1], [(0, 3, W)], 1)[0] == ERR_SHAPE
    assert versions(L, [0, 1], [0, 1], [(2, 0, W)], 1)[0] == ERR_SHAPE
    assert L.pgemm_plan_versions(2, None, None, 0, None, 0, None) == ERR_NULL


# ------------------------------------------------------------ arena

def golden_rows():
    rows = []
    for line in open(os.path.join(HERE, "golden", "tilelang_buffer_model.txt")):
        if line.startswith("#") or not line.strip():
            continue
        name, stages, no_reuse, ar, budget, verdict = line.split()
        rows.append((name, int(stages), float(no_reuse), float(ar), float(budget), verdict))
    return rows


@pytest.mark.parametrize("row", golden_rows(), ids=lambda r: f"{r[0]}-S{r[1]}")
def test_arena_reproduces_the_page_model(L, row):
    name, S, no_reuse, ar, budget, verdict = row
    loop, epi = (0, 1), (1, 2)
    if name == "epilogue":
        blocks = [(16 * KIB, S, 16, *loop), (16 * KIB, S, 16, *loop), (32 * KIB, 1, 16, *epi)]  # A, B, C
    else:
        blocks = [(16 * KIB, S, 16, *loop), (16 * KIB, S, 16, *loop), (16 * KIB, S, 16, *loop)]  # A, B, S
    a, s, offs = arena(L, blocks)
    assert s == no_reuse * KIB and a == ar * KIB
    assert ("OK" if a <= budget * KIB else "OVER") == verdict
    if name == "epilogue":
        assert offs == [0, 32 * KIB, 0]  # A at 0, B at 32 KiB, C reuses A's space


def test_arena_basic_properties(L):
    # disjoint lifetimes share space; overlapping ones never overlap in space
    a, s, offs = arena(L, [(100, 1, 16, 0, 1), (200, 1, 16, 1, 2), (50, 1, 16, 2, 3)])
    assert a == 200 and s == 350 and offs == [0, 0, 0]  # each reuses the freed top hole
    blocks = [(48, 2, 16, 0, 3), (64, 1, 64, 1, 2), (16, 1, 16, 2, 4), (128, 1, 16, 3, 5), (8, 3, 8, 0, 5)]
    a, s, offs = arena(L, blocks)
    for i, (bi, vi, ai, si, ei) in enumerate(blocks):
        assert offs[i] % ai == 0 and offs[i] + bi * vi <= a
        for j, (bj, vj, aj, sj, ej) in enumerate(blocks[:i]):
            if si < ej and sj < ei:  # live together: disjoint in space
                assert offs[i] + bi * vi <= offs[j] or offs[j] + bj * vj <= offs[i]
    assert a <= s


def test_arena_rejects(L):
    offs = (ctypes.c_int64 * 1)()
    a, s = ctypes.c_int64(), ctypes.c_int64()
    for bad in [(-1, 1, 16, 0, 1), (16, 0, 16, 0, 1), (16, 1, 12, 0, 1), (16, 1, 16, 1, 1)]:
        arr = (Block * 1)(Block(*bad))
        assert L.pgemm_plan_arena(1, arr, offs, ctypes.byref(a), ctypes.byref(s)) == ERR_SHAPE
    assert L.pgemm_plan_arena(1, None, offs, ctypes.byref(a), ctypes.byref(s)) == ERR_NULL


# ------------------------------------------------- the shipped instances

@pytest.mark.parametrize("op", ["nt_swap", "nt_ws"])
@pytest.mark.parametrize("tile", [128, 256])
@pytest.mark.parametrize("S", [1, 2, 3, 4])
def test_every_instance_fits_the_gfx950_budget(L, op, tile, S):
    # the library sizes each kernel's LDS with the planner (ring of S
    # versions, then the staging tile in the ring's space, then the credit
    # counters) and checks it against the 160 KiB of LDS a workgroup may use
    pgemm.pgemm_set_tiling(tile, 0)
    try:
        q = pgemm.pgemm_query(op, S, 4096, 4096, 4096)
    finally:
        pgemm.pgemm_set_tiling(0, 0)
    slot = (q["block_m"] + q["block_n"]) * q["block_k"] * 2
    staging = q["block_m"] * (q["block_n"] * 2 + 16)
    ctr = 2 * S * 4 if op == "nt_ws" else 0
    a, s, offs = arena(L, [(slot, S, 16, 0, 1), (staging, 1, 16, 1, 2)])
    assert q["lds_bytes"] == a + ctr == max(S * slot, staging) + ctr
    assert q["lds_bytes"] <= 160 * KIB
