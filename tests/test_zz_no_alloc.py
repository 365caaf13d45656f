"""The entry point that allocates nothing, pgemm_f16_nt_ws_static, against
pgemm_f16_nt_ws on the same operands: for callers that cannot allocate
device memory, a K-split plan keeps its fp32 partial sums in the library's
static per-device scratch instead of a workspace the caller registers.
Called through the C ABI; the same plan must give the same bits, and both
must be inside the oracle's bound (|gpu - ref| <= 1e-3 * sum_k |a*b| +
ulp(RNE(ref))) on every element.  Two calls in a row, the second smaller,
so that the second runs on what the first left in the scratch."""
import contextlib
import ctypes

import numpy as np
import pytest

import oracle
from software_pipelined_tiled_pipeline_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

STATIC_SCRATCH_BYTES = 16 << 20
ERR_WORKSPACE = 9


@pytest.fixture(scope="module")
def pg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from software_pipelined_tiled_pipeline_amd import pgemm
    pgemm.lib()
    return pgemm


@contextlib.contextmanager
def tiling(pg, tile, split):
    pg.pgemm_set_tiling(tile, split)
    try:
        yield
    finally:
        pg.pgemm_set_tiling(0, 0)


def dev_half(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.float16)


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def call(pg, name, dA, dB, out, stages, stream):
    M, K = dA.shape
    N = dB.shape[0]
    return getattr(pg.lib(), name)(ctypes.c_void_p(dA.data_ptr()), ctypes.c_void_p(dB.data_ptr()),
                                   ctypes.c_void_p(out.data_ptr()), M, N, K, stages,
                                   ctypes.c_void_p(stream.cuda_stream))


def test_static_scratch_matches_registered_workspace(pg):
    # the skinny workload (planned split in 4 pieces, 16 MiB of partial
    # sums), then a smaller split product on the same scratch
    cases = [(128, 8192, 16384, 5, 3), (64, 1000, 4096, 6, 2)]
    stream = torch.cuda.current_stream()
    prepared = []
    for M, N, K, seed, stages in cases:
        A, B = inputs.make_operands("f16_nt", M, N, K, inputs.workload_seed(seed) if seed == 5 else 900 + seed)
        q = pg.pgemm_query("nt_ws", stages, M, N, K)
        assert q["k_split"] > 1 and 0 < q["workspace_bytes"] <= STATIC_SCRATCH_BYTES
        prepared.append((A, B, dev_half(A), dev_half(B), stages, q))
    # the existing entry point with a registered workspace of the plan's size
    want = []
    for A, B, dA, dB, stages, q in prepared:
        pg.ensure_workspace(q["workspace_bytes"], stream)
        out = torch.empty((dA.shape[0], dB.shape[0]), dtype=torch.float16, device="cuda")
        assert call(pg, "pgemm_f16_nt_ws", dA, dB, out, stages, stream) == 0
        torch.cuda.synchronize()
        want.append(host_bits(out))
    pg.release_workspace(stream)
    outs = [torch.full((dA.shape[0], dB.shape[0]), 7.0, dtype=torch.float16, device="cuda")
            for _, _, dA, dB, _, _ in prepared]
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for (A, B, dA, dB, stages, q), out in zip(prepared, outs):
        assert call(pg, "pgemm_f16_nt_ws_static", dA, dB, out, stages, stream) == 0
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0, "the static entry point changed the free device memory"
    assert pg.pgemm_debug_status() == 0
    for (A, B, dA, dB, stages, q), out, w in zip(prepared, outs, want):
        got = host_bits(out)
        assert np.array_equal(got, w), f"{A.shape[0]}x{B.shape[0]}x{A.shape[1]}: differs from pgemm_f16_nt_ws"
        ref, mag = oracle.gemm_nt("f16", A, B)
        bad, worst = oracle.check_nt("f16", got, ref, mag)
        assert bad == 0, f"{bad} elements outside the bound (worst err/bound {worst:.3g})"


def test_static_scratch_unsplit_and_too_large(pg):
    stream = torch.cuda.current_stream()
    # an unsplit plan does not touch the scratch
    A, B = inputs.make_operands("f16_nt", 300, 260, 136, 17)
    dA, dB = dev_half(A), dev_half(B)
    out = torch.empty((300, 260), dtype=torch.float16, device="cuda")
    assert pg.pgemm_query("nt_ws", 0, 300, 260, 136)["k_split"] == 1
    assert call(pg, "pgemm_f16_nt_ws_static", dA, dB, out, 0, stream) == 0
    torch.cuda.synchronize()
    ref, mag = oracle.gemm_nt("f16", A, B)
    assert oracle.check_nt("f16", host_bits(out), ref, mag)[0] == 0
    # a forced split whose partial sums exceed the scratch is refused
    M, N, K = 1024, 1024, 4096
    dA = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    dB = torch.zeros((N, K), dtype=torch.float16, device="cuda")
    out = torch.full((M, N), 3.0, dtype=torch.float16, device="cuda")
    with tiling(pg, 128, 8):
        assert pg.pgemm_query("nt_ws", 0, M, N, K)["workspace_bytes"] > STATIC_SCRATCH_BYTES
        assert call(pg, "pgemm_f16_nt_ws_static", dA, dB, out, 0, stream) == ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 3.0).item(), "a refused call must enqueue nothing"
