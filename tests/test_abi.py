"""The C-ABI library on the CPU: it loads, exports every symbol its header
declares, plans launches, and rejects bad arguments before any HIP call.
Nothing here launches a kernel."""
import ctypes
import os
import re

import pytest

from software_pipelined_tiled_pipeline_amd import pgemm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pgemm.h")

OK, ERR_NULL, ERR_SHAPE, ERR_STAGES, ERR_ALIGN, ERR_LDS = 0, 1, 2, 3, 4, 5


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(pgemm.LIB_PATH):
        pytest.fail("libpgemm.so is not built (run __graft_entry__.build())")
    return pgemm.lib()


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pgemm_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n


def test_version_and_messages(L):
    assert pgemm.abi_version() == 3
    for code in range(10):
        assert pgemm.strerror(code) and pgemm.strerror(code) != "unknown status"
    assert pgemm.strerror(99) == "unknown status"


def test_query_geometry(L):
    q = pgemm.pgemm_query("s32_nn", 0, 128, 256, 256)
    assert (q["block_m"], q["block_n"], q["block_k"], q["stages"]) == (16, 16, 16, 2)
    assert q["grid"] == 8 * 16 and q["threads"] == 256 and q["k_tiles"] == 16
    q = pgemm.pgemm_query("nt_swap", 0, 8192, 8192, 8192)
    assert q["stages"] == 2 and q["producer_waves"] == 0
    assert q["grid"] == (8192 // q["block_m"]) * (8192 // q["block_n"])
    for s in (1, 2, 3, 4):
        q = pgemm.pgemm_query("nt_ws", s, 4095, 1000, 1000)
        assert q["stages"] == s and q["producer_waves"] > 0 and q["consumer_waves"] > 0
        assert q["lds_bytes"] <= 160 * 1024
        assert q["threads"] == 64 * (q["producer_waves"] + q["consumer_waves"])
        assert q["k_tiles"] == -(-1000 // q["block_k"])
        # the ring holds `stages` versions of the (A, B) tile pair
        ring = s * (q["block_m"] + q["block_n"]) * q["block_k"] * 2
        assert ring <= q["lds_bytes"]
    assert pgemm.pgemm_query("nt_ws", 0, 64, 64, 64)["stages"] == 4


def cdiv(a, b):
    return -(-a // b)


@pytest.mark.parametrize("op", ["nt_swap", "nt_ws"])
def test_planner_on_the_workloads(L, op):
    # 8192^3 and 4096^3: 1024 and 256 large tiles, enough to fill the chip
    for n in (8192, 4096):
        q = pgemm.pgemm_query(op, 0, n, n, n)
        assert (q["block_m"], q["block_n"], q["k_split"]) == (256, 256, 1)
        assert q["persistent"] == 0
        assert q["grid"] == (n // 256) ** 2 and q["workspace_bytes"] == 0
    # ragged bf16 4095 x 1000 x 1000: 64 large tiles, so small ones (256)
    q = pgemm.pgemm_query(op, 0, 4095, 1000, 1000)
    assert (q["block_m"], q["block_n"], q["k_split"], q["grid"]) == (128, 128, 1, 32 * 8)
    # skinny 128 x 8192 x 16384: 64 small tiles, K split in 4 pieces of 4096
    q = pgemm.pgemm_query(op, 0, 128, 8192, 16384)
    assert (q["block_m"], q["block_n"], q["k_split"], q["grid"]) == (128, 128, 4, 256)
    assert q["k_tiles"] == 4096 // 64
    assert q["workspace_bytes"] == 4 * 128 * 8192 * 4


@pytest.mark.parametrize("M,N,K", [(1, 1, 8), (128, 128, 1024), (100, 300, 1000), (64, 64, 4096), (7, 9000, 2 ** 21),
                                   (2000, 2000, 64), (256, 768, 40000)])
@pytest.mark.parametrize("force", [(0, 0), (128, 0), (128, 1), (128, 2), (128, 3), (128, 16), (256, 0)])
def test_planner_invariants(L, M, N, K, force):
    pgemm.pgemm_set_tiling(*force)
    try:
        for op in ("nt_swap", "nt_ws"):
            q = pgemm.pgemm_query(op, 0, M, N, K)
            if force[0]:
                assert q["block_m"] == q["block_n"] == force[0]
            split = q["k_split"]
            assert split >= 1 and q["grid"] == cdiv(M, q["block_m"]) * cdiv(N, q["block_n"]) * split
            if split == 1:
                assert q["k_tiles"] == cdiv(K, q["block_k"]) and q["workspace_bytes"] == 0
            else:
                assert q["block_m"] == 128 and (force[1] == 0 or split <= force[1])
                chunk = q["k_tiles"] * q["block_k"]
                assert chunk % 64 == 0
                assert (split - 1) * chunk < K <= split * chunk  # no empty piece
                assert q["workspace_bytes"] == split * M * (cdiv(N, 4) * 4) * 4
            if force[1] == 1:
                assert split == 1
            assert q["lds_bytes"] <= 160 * 1024
    finally:
        pgemm.pgemm_set_tiling(0, 0)


@pytest.mark.parametrize("M,N,K", [(8192, 8192, 8192), (4096, 4096, 64), (300, 200, 1000), (2560, 2048, 136),
                                   (128, 8192, 16384)])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_persistent_schedule_plan(L, M, N, K, mode):
    pgemm.pgemm_set_persistent(mode)
    try:
        for S in (1, 2, 3, 4):
            q = pgemm.pgemm_query("nt_ws", S, M, N, K)
            tiles = cdiv(M, q["block_m"]) * cdiv(N, q["block_n"])
            if q["k_split"] > 1:
                assert q["persistent"] == 0  # split products keep the per-tile kernel
                continue
            expect = mode == 2
            assert q["persistent"] == int(expect)
            if expect:
                per_cu = min(2, (160 * 1024) // q["lds_bytes"])
                assert q["grid"] == min(tiles, 256 * per_cu)
            else:
                assert q["grid"] == tiles
            assert pgemm.pgemm_query("nt_swap", S, M, N, K)["persistent"] == 0
    finally:
        pgemm.pgemm_set_persistent(0)
    assert L.pgemm_set_persistent(3) == ERR_SHAPE and L.pgemm_set_persistent(-1) == ERR_SHAPE


def test_set_tiling_rejects(L):
    for tile, split in [(100, 0), (64, 0), (256, 2), (0, 2), (0, 17), (128, -1), (128, 17)]:
        assert L.pgemm_set_tiling(tile, split) == ERR_SHAPE
    assert pgemm.pgemm_query("nt_ws", 0, 8192, 8192, 8192)["block_m"] == 256  # nothing changed


@pytest.mark.parametrize("op,stages", [("s32_nn", 3), ("nt_swap", 5), ("nt_ws", 5), ("nt_ws", -1)])
def test_query_rejects_stages(L, op, stages):
    info = pgemm.KernelInfo()
    assert L.pgemm_query(pgemm.OPS[op], stages, 64, 64, 64, ctypes.byref(info)) == ERR_STAGES


def test_query_rejects_shapes(L):
    info = pgemm.KernelInfo()
    assert L.pgemm_query(1, 0, -1, 64, 64, ctypes.byref(info)) == ERR_SHAPE
    assert L.pgemm_query(1, 0, 64, 2 ** 31, 64, ctypes.byref(info)) == ERR_SHAPE
    assert L.pgemm_query(1, 0, 64, 64, 2 ** 31, ctypes.byref(info)) == ERR_SHAPE
    for op in (0, 1, 2):  # any K below 2^31
        assert L.pgemm_query(op, 0, 64, 64, 2 ** 31 - 1, ctypes.byref(info)) == OK
    assert L.pgemm_query(1, 0, 64, 64, 64, None) == ERR_NULL


def test_grid_limits(L):
    # A dispatch counts its work-items in 32 bits.  int32: one workgroup per
    # 16 x 16 tile up to 2^20, beyond that 2^20 workgroups walk the tiles.
    q = pgemm.pgemm_query("s32_nn", 0, 100, 100, 8)
    assert q["grid"] == 7 * 7
    assert pgemm.pgemm_query("s32_nn", 0, 16384, 16384, 8)["grid"] == 1 << 20
    assert pgemm.pgemm_query("s32_nn", 0, 16400, 16400, 8)["grid"] == 1 << 20
    assert pgemm.pgemm_query("s32_nn", 0, 2 ** 31 - 1, 2 ** 31 - 1, 8)["grid"] == 1 << 20
    # NT: a plan of 2^32 work-items or more is refused, one just below is not
    info = pgemm.KernelInfo()
    n = 2 ** 31 - 1
    assert L.pgemm_query(pgemm.OPS["nt_ws"], 0, n, n, 8, ctypes.byref(info)) == ERR_SHAPE
    pgemm.pgemm_set_tiling(128, 1)
    try:
        # 128 x 128 tiles of 512 (swap) or 384 (ws) threads
        for op, threads in (("nt_swap", 512), ("nt_ws", 384)):
            tiles_limit = -(-(2 ** 32) // threads)  # the first tile count that reaches 2^32
            m = 128 * ((tiles_limit - 1) // 4096)  # 4096 tile columns, as many tile rows as fit
            assert L.pgemm_query(pgemm.OPS[op], 0, m, 128 * 4096, 8, ctypes.byref(info)) == OK
            assert info.grid * info.threads < 2 ** 32
            m = 128 * cdiv(tiles_limit, 4096)
            assert L.pgemm_query(pgemm.OPS[op], 0, m, 128 * 4096, 8, ctypes.byref(info)) == ERR_SHAPE
    finally:
        pgemm.pgemm_set_tiling(0, 0)


FAKE = 0x7F0000000000  # never dereferenced: every case below fails validation first


@pytest.mark.parametrize("name", pgemm.GEMM_SYMBOLS)
def test_argument_errors_before_any_hip_call(L, name):
    f = getattr(L, name)
    nt = name != "pgemm_s32_nn"
    assert f(None, FAKE, FAKE, 64, 64, 64, 0, None) == ERR_NULL
    assert f(FAKE, None, FAKE, 64, 64, 64, 0, None) == ERR_NULL
    assert f(FAKE, FAKE, None, 64, 64, 64, 0, None) == ERR_NULL
    assert f(FAKE + 2, FAKE, FAKE, 64, 64, 64, 0, None) == ERR_ALIGN
    assert f(FAKE, FAKE, FAKE + 8, 64, 64, 64, 0, None) == ERR_ALIGN
    assert f(FAKE, FAKE, FAKE, -1, 64, 64, 0, None) == ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 64, 64, 2 ** 31, 0, None) == ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 64, 64, 64, 7, None) == ERR_STAGES
    # empty outputs: nothing to launch; pointers to empty matrices may be NULL
    assert f(None, FAKE, None, 0, 64, 64, 0, None) == OK
    assert f(FAKE, None, None, 64, 0, 64, 0, None) == OK
    assert f(None, None, None, 0, 0, 64, 0, None) == OK


@pytest.mark.parametrize("op", ["nt_swap", "nt_ws"])
def test_loader_choice(L, op):
    # 16-byte direct-to-LDS loads when every row starts on 16 bytes and a
    # tile's rows span less than 2^31 bytes; the staged loader otherwise
    for K in (8, 1000, 4096, 8192):
        assert pgemm.pgemm_query(op, 0, 8192, 8192, K)["staged"] == 0
    for K in range(1, 16):
        assert pgemm.pgemm_query(op, 0, 300, 200, K)["staged"] == int(K % 8 != 0)
    for K in (1001, 4095, 2 ** 22 + 1):
        assert pgemm.pgemm_query(op, 0, 4095, 1000, K)["staged"] == 1
    # panel span: tile * K < 2^30 elements
    pgemm.pgemm_set_tiling(256, 1)
    try:
        assert pgemm.pgemm_query(op, 0, 256, 256, 2 ** 22 - 8)["staged"] == 0
        assert pgemm.pgemm_query(op, 0, 256, 256, 2 ** 22)["staged"] == 1
    finally:
        pgemm.pgemm_set_tiling(0, 0)
    pgemm.pgemm_set_tiling(128, 1)
    try:
        assert pgemm.pgemm_query(op, 0, 256, 256, 2 ** 22)["staged"] == 0
        assert pgemm.pgemm_query(op, 0, 256, 256, 2 ** 23)["staged"] == 1
    finally:
        pgemm.pgemm_set_tiling(0, 0)


def test_staged_plans_keep_the_per_tile_kernel(L):
    pgemm.pgemm_set_persistent(2)
    try:
        assert pgemm.pgemm_query("nt_ws", 0, 8192, 8192, 8192)["persistent"] == 1
        q = pgemm.pgemm_query("nt_ws", 0, 8192, 8192, 8190)
        assert q["staged"] == 1 and q["persistent"] == 0
    finally:
        pgemm.pgemm_set_persistent(0)


def test_set_workspace_argument_errors(L):
    # checked before any HIP call
    assert L.pgemm_set_workspace(None, FAKE, -1) == ERR_SHAPE
    assert L.pgemm_set_workspace(None, None, 64) == ERR_NULL
    assert L.pgemm_set_workspace(None, FAKE + 4, 64) == ERR_ALIGN
