"""GPU parity of the register-staged loader and of the caller-owned K-split
workspace.

The staged loader fills the LDS ring from 64-bit addressed loads, guarded
element by element, whenever the 16-byte direct-to-LDS loads cannot be used:
K not a multiple of 8 (rows do not start on 16 bytes), or a tile's rows
spanning 2^31 bytes or more.  Every case is compared with the oracle over the
whole output (|gpu - ref| <= 1e-3 * sum_k |a*b| + ulp(RNE(ref))), and with
the direct path on the same operands zero-padded to the next multiple of 8:
the padding adds exact zeros to the same MFMA steps, so the bits must agree.
"""
import contextlib
import ctypes
import threading

import numpy as np
import pytest

import oracle
from software_pipelined_tiled_pipeline_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

VARIANTS = [("swap", 1), ("swap", 2), ("swap", 3), ("swap", 4), ("ws", 1), ("ws", 2), ("ws", 3), ("ws", 4)]


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


def dev_half(bits, fmt):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return t.view(torch.float16 if fmt == "f16" else torch.bfloat16)


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_nt(pg, fmt, variant, dA, dB, stages, **kw):
    name = f"pgemm_{fmt}_nt" + ("_ws" if variant == "ws" else "")
    out = getattr(pg, name)(dA, dB, stages=stages, **kw)
    torch.cuda.synchronize()
    return host_bits(out)


def assert_within_bound(fmt, got, ref, mag, what):
    bad, worst = oracle.check_nt(fmt, got, ref, mag)
    assert bad == 0, f"{what}: {bad} elements outside the bound (worst err/bound {worst:.3g})"


def pad8(bits):
    K = bits.shape[1]
    K8 = -(-K // 8) * 8
    out = np.zeros((bits.shape[0], K8), np.uint16)
    out[:, :K] = bits
    return out


KS = [1, 2, 3, 4, 5, 6, 7, 9, 15, 1001, 4095]


@pytest.mark.parametrize("tile", [128, 256])
@pytest.mark.parametrize("K", KS)
def test_k_not_multiple_of_8_every_variant(pg, K, tile):
    # several output tiles with ragged edges; K from one element up to many
    # K tiles with a tail of every length mod 8
    M, N = 300, 260
    fmt = "f16" if K % 2 else "bf16"
    kind = fmt + "_nt"
    A, B = inputs.make_operands(kind, M, N, K, 500 + K)
    ref, mag = oracle.gemm_nt(fmt, A, B)
    dA, dB = dev_half(A, fmt), dev_half(B, fmt)
    with tiling(pg, tile, 1):
        q = pg.pgemm_query("nt_ws", 0, M, N, K)
        assert q["staged"] == 1 and q["block_m"] == tile and q["k_split"] == 1
        first = None
        for variant, s in VARIANTS:
            got = run_nt(pg, fmt, variant, dA, dB, s)
            what = f"{fmt} {variant} S={s} tile {tile} {M}x{N}x{K}"
            assert_within_bound(fmt, got, ref, mag, what)
            if first is None:
                first = got
            else:
                assert np.array_equal(got, first), f"{what} differs in bits from swap S=1"
        # the direct path on zero-padded operands: same MFMA steps, same bits
        pA, pB = dev_half(pad8(A), fmt), dev_half(pad8(B), fmt)
        assert pg.pgemm_query("nt_ws", 0, M, N, pA.shape[1])["staged"] == 0
        for variant, s in (("swap", 2), ("ws", 3)):
            assert np.array_equal(run_nt(pg, fmt, variant, pA, pB, s), first), f"padded direct {variant} S={s}"


@pytest.mark.parametrize("K", [4095, 3001])
def test_k_not_multiple_of_8_split(pg, K):
    # a K split with a ragged last piece: the pieces are multiples of 64,
    # the tail of the last one is guarded element by element
    M, N = 200, 1000
    A, B = inputs.make_operands("f16_nt", M, N, K, 600 + K)
    ref, mag = oracle.gemm_nt("f16", A, B)
    dA, dB = dev_half(A, "f16"), dev_half(B, "f16")
    pA, pB = dev_half(pad8(A), "f16"), dev_half(pad8(B), "f16")
    with tiling(pg, 128, 3):
        q = pg.pgemm_query("nt_ws", 0, M, N, K)
        assert q["staged"] == 1 and q["k_split"] == 3
        assert pg.pgemm_query("nt_ws", 0, M, N, pA.shape[1])["k_split"] == 3
        for variant, s in VARIANTS:
            got = run_nt(pg, "f16", variant, dA, dB, s)
            assert_within_bound("f16", got, ref, mag, f"split {variant} S={s}")
            assert np.array_equal(got, run_nt(pg, "f16", variant, pA, pB, s)), f"padded split {variant} S={s}"


def test_k_not_multiple_of_8_planned(pg):
    # the planner's own choice (large tiles here) on a shape of many tiles
    M, N, K = 1300, 1100, 999
    A, B = inputs.make_operands("bf16_nt", M, N, K, 77)
    ref, mag = oracle.gemm_nt("bf16", A, B)
    dA, dB = dev_half(A, "bf16"), dev_half(B, "bf16")
    for variant, s in (("swap", 2), ("ws", 4)):
        assert_within_bound("bf16", run_nt(pg, "bf16", variant, dA, dB, s), ref, mag, f"planned {variant}")


def device_f16(rows, cols, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = torch.empty((rows, cols), dtype=torch.float16, device="cuda")
    for r in range(0, rows, 8):
        n = min(8, rows - r)
        out[r:r + n] = (torch.rand((n, cols), generator=g, device="cuda") * 2 - 1).half()
    return out


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("M,N,K,tile,split,staged", [
    (256, 8, (1 << 22) + 8, 256, 1, 1),   # 256-row panels past 2^31 bytes: staged
    (256, 8, (1 << 22) + 8, 128, 1, 0),   # 128-row panels still within reach: direct
    (256, 8, (1 << 22) + 8, 0, 0, 0),     # the planner's K split (direct)
    (64, 8, (1 << 23) + 8, 128, 1, 1),    # 128-row panels past 2^31 bytes: staged
    (40, 24, (1 << 22) + 7, 0, 0, 1),     # long and not a multiple of 8, split
])
def test_long_k(pg, M, N, K, tile, split, staged):
    # operands drawn on the device (seeded) and copied back for the oracle
    dA, dB = device_f16(M, K, 41 + M), device_f16(N, K, 42 + N)
    ref, mag = oracle.gemm_nt("f16", bits(dA), bits(dB))
    with tiling(pg, tile, split):
        for name, op, s in (("pgemm_f16_nt", "nt_swap", 2), ("pgemm_f16_nt_ws", "nt_ws", 4)):
            q = pg.pgemm_query(op, s, M, N, K)
            assert q["staged"] == staged
            out = getattr(pg, name)(dA, dB, stages=s)
            torch.cuda.synchronize()
            assert_within_bound("f16", bits(out), ref, mag, f"{name} S={s} K={K} tile={tile} split={q['k_split']}")
    del dA, dB
    torch.cuda.empty_cache()


# ------------------------------------------------ caller-owned workspace

def _raw_call(pg, name, dA, dB, out, stream):
    M, K = dA.shape
    N = dB.shape[0]
    f = getattr(pg.lib(), name)
    st = f(ctypes.c_void_p(dA.data_ptr()), ctypes.c_void_p(dB.data_ptr()), ctypes.c_void_p(out.data_ptr()),
           M, N, K, 0, ctypes.c_void_p(stream.cuda_stream))
    assert st == 0, pg.strerror(st)


def test_split_needs_a_registered_workspace(pg):
    # Without a registered workspace a call whose plan splits K runs the same
    # tiling unsplit; with one it splits, and allocates nothing itself.
    M, N, K = 128, 1024, 8192
    A, B = inputs.make_operands("f16_nt", M, N, K, 31)
    ref, mag = oracle.gemm_nt("f16", A, B)
    dA, dB = dev_half(A, "f16"), dev_half(B, "f16")
    q = pg.pgemm_query("nt_ws", 0, M, N, K)
    assert q["k_split"] > 1 and q["workspace_bytes"] > 0
    s = torch.cuda.Stream()
    out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    pg.release_workspace(s)
    with tiling(pg, 128, 1):
        unsplit = run_nt(pg, "f16", "ws", dA, dB, 0, split=False)
    _raw_call(pg, "pgemm_f16_nt_ws", dA, dB, out, s)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), unsplit), "no workspace: the unsplit plan"
    # too small: unsplit too
    small = torch.empty(q["workspace_bytes"] - 16, dtype=torch.uint8, device="cuda")
    assert pg.lib().pgemm_set_workspace(ctypes.c_void_p(s.cuda_stream), ctypes.c_void_p(small.data_ptr()),
                                        small.numel()) == 0
    _raw_call(pg, "pgemm_f16_nt_ws", dA, dB, out, s)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), unsplit), "small workspace: the unsplit plan"
    # large enough: the split plan, no device memory taken by the call
    big = torch.empty(q["workspace_bytes"], dtype=torch.uint8, device="cuda")
    assert pg.lib().pgemm_set_workspace(ctypes.c_void_p(s.cuda_stream), ctypes.c_void_p(big.data_ptr()),
                                        big.numel()) == 0
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    _raw_call(pg, "pgemm_f16_nt_ws", dA, dB, out, s)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0, "the call changed the free device memory"
    split = host_bits(out)
    assert not np.array_equal(split, unsplit)  # a different summation order in the last bits
    assert_within_bound("f16", split, ref, mag, "split")
    with tiling(pg, 128, q["k_split"]):
        assert np.array_equal(run_nt(pg, "f16", "ws", dA, dB, 0), split)
    assert pg.lib().pgemm_set_workspace(ctypes.c_void_p(s.cuda_stream), None, 0) == 0
    del small, big


def test_split_calls_from_two_threads_on_one_stream(pg):
    # Two host threads enqueue K-split products on the same stream, sharing
    # its workspace: each call's GEMM and reduction stay adjacent in the
    # stream, so every result is its own product's.
    shapes = [(128, 1000, 8192), (64, 2048, 4096)]
    data = []
    for i, (M, N, K) in enumerate(shapes):
        A, B = inputs.make_operands("f16_nt", M, N, K, 70 + i)
        data.append((dev_half(A, "f16"), dev_half(B, "f16"), *oracle.gemm_nt("f16", A, B)))
    s = torch.cuda.Stream()
    need = max(pg.pgemm_query("nt_ws", 0, d[0].shape[0], d[1].shape[0], d[0].shape[1])["workspace_bytes"]
               for d in data)
    pg.ensure_workspace(need, s)
    outs = [[torch.empty((d[0].shape[0], d[1].shape[0]), dtype=torch.float16, device="cuda") for _ in range(20)]
            for d in data]
    torch.cuda.synchronize()

    def worker(i):
        dA, dB = data[i][0], data[i][1]
        for o in outs[i]:
            _raw_call(pg, "pgemm_f16_nt_ws" if i else "pgemm_f16_nt", dA, dB, o, s)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for i, (_, _, ref, mag) in enumerate(data):
        first = host_bits(outs[i][0])
        assert_within_bound("f16", first, ref, mag, f"thread {i}")
        for o in outs[i][1:]:
            assert np.array_equal(host_bits(o), first), f"thread {i}: a result differs"
    pg.release_workspace(s)


# ------------------------------------------------ binding argument checks

def test_binding_rejects_tensors_off_the_current_device(pg):
    # host tensors (or tensors on another device) are refused in Python,
    # before any pointer reaches the library
    dA = torch.zeros((64, 32), dtype=torch.float16, device="cuda")
    dB = torch.zeros((48, 32), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        pg.pgemm_f16_nt_ws(dA, dB, out=torch.zeros((64, 48), dtype=torch.float16))
    with pytest.raises(ValueError):
        pg.pgemm_f16_nt(dA.cpu(), dB)
    with pytest.raises(ValueError):
        pg.pgemm_bf16_nt(dA.bfloat16(), dB.bfloat16().cpu())
    with pytest.raises(ValueError):
        pg.pgemm_f16_nt_ws_static(dA, dB, out=torch.zeros((64, 48), dtype=torch.float16))
    with pytest.raises(ValueError):
        pg.pgemm_s32_nn(torch.zeros((4, 4), dtype=torch.int32), torch.zeros((4, 4), dtype=torch.int32, device="cuda"))
    out = pg.pgemm_f16_nt_ws(dA, dB)  # the same call on device tensors runs
    torch.cuda.synchronize()
    assert out.is_cuda and torch.count_nonzero(out).item() == 0
