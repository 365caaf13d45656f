"""GPU parity at the size limits of the C ABI: an int32 product with more
output tiles than the int32 kernel's grid holds, an f16 product whose lhs
spans more than 4 GiB (row offsets past 2^31 elements), one whose output has
more than 2^31 elements, and the longest K the NT calls accept.  Operands
too large to generate on the host are drawn on the device; the rows the
checks need are copied back and handed to the oracle.  int32 is compared bit
for bit, f16 within |gpu - ref| <= 1e-3 * sum_k |a*b| + ulp(RNE(ref))."""
import numpy as np
import pytest

import oracle
from software_pipelined_tiled_pipeline_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MAX_K_NT = (1 << 22) - 8  # the longest K (a multiple of 8 below 2^22)


@pytest.fixture(scope="module")
def pg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from software_pipelined_tiled_pipeline_amd import pgemm
    pgemm.lib()
    return pgemm


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def device_f16(rows, cols, seed, chunk_rows=1 << 16):
    """Uniform [-1, 1) f16 drawn on the device, in row chunks so that the
    fp32 draw never holds more than a chunk."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = torch.empty((rows, cols), dtype=torch.float16, device="cuda")
    for r in range(0, rows, chunk_rows):
        n = min(chunk_rows, rows - r)
        out[r:r + n] = (torch.rand((n, cols), generator=g, device="cuda") * 2 - 1).half()
    return out


def check_rows(pg, out, dA, dB, rows, what):
    rows_t = torch.as_tensor(rows, device="cuda")
    ref, mag = oracle.gemm_nt("f16", bits(dA[rows_t]), bits(dB))
    bad, worst = oracle.check_nt("f16", bits(out[rows_t]), ref, mag)
    assert bad == 0, f"{what}: {bad} elements outside the bound (worst err/bound {worst:.3g})"


def test_s32_more_output_tiles_than_workgroups(pg):
    # 1025 x 1025 tiles of 16 x 16: workgroup b takes tiles b and b + 2^20,
    # the second pass covering the last two column tiles
    M, N, K = 16400, 16400, 21
    assert pg.pgemm_query("s32_nn", 0, M, N, K)["grid"] == 1 << 20
    A, B = inputs.make_operands("s32_nn", M, N, K, 77)
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    rng = np.random.default_rng(1)
    rows = np.concatenate([np.arange(16), np.arange(M - 16, M), rng.integers(0, M, 32)])
    ref_rows = oracle.gemm_s32_nn(A[rows], B)
    ref_cols = oracle.gemm_s32_nn(A, np.ascontiguousarray(B[:, -48:]))
    for s in (1, 2):
        out = pg.pgemm_s32_nn(dA, dB, stages=s)
        torch.cuda.synchronize()
        assert np.array_equal(out[torch.as_tensor(rows).cuda()].cpu().numpy(), ref_rows), f"S={s} rows"
        assert np.array_equal(out[:, -48:].cpu().numpy(), ref_cols), f"S={s} last columns"
        del out


def test_f16_lhs_past_4gib(pg):
    # lhs is 4.3 GB: the panels of the last row tiles start past 2^31
    # elements (and 2^32 bytes) from its base
    M, N, K = (1 << 19) + 37, 72, 4104
    dA = device_f16(M, K, 11)
    dB = device_f16(N, K, 12)
    assert pg.pgemm_query("nt_ws", 0, M, N, K)["k_split"] == 1
    rng = np.random.default_rng(2)
    rows = np.concatenate([np.arange(8), np.arange(M - 300, M), rng.integers(0, M, 40)])
    for name, s in (("pgemm_f16_nt", 2), ("pgemm_f16_nt_ws", 4)):
        out = getattr(pg, name)(dA, dB, stages=s)
        torch.cuda.synchronize()
        check_rows(pg, out, dA, dB, rows, f"{name} S={s}")
        del out
    del dA, dB
    torch.cuda.empty_cache()


def test_f16_output_past_2g_elements(pg):
    # out has 2^21 + 5 rows of 1032: 2.16e9 elements, so its last rows start
    # past 2^31 elements
    M, N, K = (1 << 21) + 5, 1032, 16
    dA = device_f16(M, K, 21)
    dB = device_f16(N, K, 22)
    rng = np.random.default_rng(3)
    rows = np.concatenate([np.arange(4), np.arange(M - 260, M), rng.integers(0, M, 24)])
    for name, s in (("pgemm_f16_nt", 2), ("pgemm_f16_nt_ws", 3)):
        out = getattr(pg, name)(dA, dB, stages=s)
        torch.cuda.synchronize()
        check_rows(pg, out, dA, dB, rows, f"{name} S={s}")
        del out
    del dA, dB
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def longest_k():
    # 256 rows of K = 2^22 - 8: a 256-row panel is 2,147,479,552 bytes, just
    # under the 2^31-byte limit of one buffer resource
    M, N, K = 256, 8, MAX_K_NT
    dA, dB = device_f16(M, K, 31, chunk_rows=8), device_f16(N, K, 32, chunk_rows=8)
    ref, mag = oracle.gemm_nt("f16", bits(dA), bits(dB))
    yield dA, dB, ref, mag
    del dA, dB
    torch.cuda.empty_cache()


@pytest.mark.parametrize("tile,split", [(0, 0), (128, 1), (256, 1)])
def test_f16_longest_k(pg, longest_k, tile, split):
    # the planner's K split (16 pieces), or one workgroup per tile walking
    # all of K in 128- or 256-row panels
    dA, dB, ref, mag = longest_k
    M, K = dA.shape
    N = dB.shape[0]
    pg.pgemm_set_tiling(tile, split)
    try:
        for name, op, s in (("pgemm_f16_nt", "nt_swap", 2), ("pgemm_f16_nt_ws", "nt_ws", 4)):
            q = pg.pgemm_query(op, s, M, N, K)
            assert (q["k_split"] == 16) if split == 0 else (q["k_split"] == 1 and q["block_m"] == tile)
            out = getattr(pg, name)(dA, dB, stages=s)
            torch.cuda.synchronize()
            bad, worst = oracle.check_nt("f16", bits(out), ref, mag)
            assert bad == 0, f"{name} S={s}: {bad} elements outside the bound (worst {worst:.3g})"
    finally:
        pg.pgemm_set_tiling(0, 0)
