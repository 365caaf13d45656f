"""Properties of the NT launch planner over random shapes, stage counts and
forced tilings, through pgemm_query on the CPU (nothing is launched): the
grid covers every output tile and K piece, pieces are whole multiples of the
small tile's K tile with none empty, the workspace holds the partial planes,
the ring fits in LDS, and a dispatch never reaches 2^32 work-items."""
import ctypes

import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

from software_pipelined_tiled_pipeline_amd import pgemm  # noqa: E402

OK, ERR_SHAPE = 0, 2
LDS_LIMIT = 160 * 1024
TILINGS = [(0, 0), (128, 0), (128, 1), (128, 2), (128, 3), (128, 7), (128, 16), (256, 0), (256, 1)]


def cdiv(a, b):
    return -(-a // b)


@settings(max_examples=400, deadline=None)
@given(M=st.integers(1, 1 << 20), N=st.integers(1, 1 << 20), K=st.integers(0, (1 << 22) - 1),
       op=st.sampled_from(["nt_swap", "nt_ws"]), stages=st.integers(0, 4), tiling=st.sampled_from(TILINGS))
def test_nt_plan_properties(M, N, K, op, stages, tiling):
    L = pgemm.lib()
    info = pgemm.KernelInfo()
    L.pgemm_set_tiling(*tiling)
    try:
        st_ = L.pgemm_query(pgemm.OPS[op], stages, M, N, K, ctypes.byref(info))
    finally:
        L.pgemm_set_tiling(0, 0)
    tile, force_split = tiling
    if st_ == ERR_SHAPE:
        # in this range only a grid of 2^32 work-items or more is refused
        bm = tile or (256 if cdiv(M, 256) * cdiv(N, 256) >= 192 else 128)
        threads = {("nt_swap", 256): 256, ("nt_swap", 128): 512, ("nt_ws", 256): 768, ("nt_ws", 128): 384}[op, bm]
        pieces = 1
        if bm == 128 and force_split > 1 and K > 0:
            pieces = cdiv(K, cdiv(cdiv(K, force_split), 64) * 64)
        assert cdiv(M, bm) * cdiv(N, bm) * pieces * threads >= 1 << 32
        return
    assert st_ == OK
    bm, bn, split = info.block_m, info.block_n, info.k_split
    assert bm == bn and bm in (128, 256)
    if tile:
        assert bm == tile
    else:
        assert (bm == 256) == (cdiv(M, 256) * cdiv(N, 256) >= 192)
    assert info.stages == (stages or (4 if op == "nt_ws" else 2))
    assert 1 <= split <= 16
    if split > 1:
        assert bm == 128 and K > 0
        if force_split:
            assert split <= force_split
        chunk = info.k_tiles * info.block_k
        assert chunk % 64 == 0
        assert (split - 1) * chunk < K <= split * chunk  # every piece holds some of K
        assert info.workspace_bytes == split * M * cdiv(N, 4) * 4 * 4
    else:
        assert info.k_tiles == cdiv(K, info.block_k) and info.workspace_bytes == 0
    assert info.grid == cdiv(M, bm) * cdiv(N, bn) * split
    assert 0 < info.lds_bytes <= LDS_LIMIT
    assert info.threads == 64 * (info.producer_waves + info.consumer_waves)
    assert (info.producer_waves > 0) == (op == "nt_ws")
    assert info.grid * info.threads < 1 << 32


@settings(max_examples=200, deadline=None)
@given(M=st.integers(1, (1 << 31) - 1), N=st.integers(1, (1 << 31) - 1), K=st.integers(0, 1 << 24), stages=st.integers(0, 2))
def test_s32_plan_properties(M, N, K, stages):
    info = pgemm.KernelInfo()
    assert pgemm.lib().pgemm_query(pgemm.OPS["s32_nn"], stages, M, N, K, ctypes.byref(info)) == OK
    tiles = cdiv(M, 16) * cdiv(N, 16)
    assert info.grid == min(tiles, 1 << 20)  # workgroups walk the tiles beyond 2^20
    assert info.grid * info.threads < 1 << 32
    assert info.k_tiles == cdiv(K, 16) and info.stages == (stages or 2)
