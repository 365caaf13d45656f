"""GPU parity: every pgemm entry point against the CPU oracle.

int32 results must be bit-exact.  f16/bf16 results must satisfy, element by
element, |gpu - ref| <= 1e-3 * sum_k |a*b| + ulp(RNE(ref)) in the output
type, with ref and sum_k |a*b| from the binary64 oracle.  Every output,
the full-size workloads included, is compared with the oracle element by
element over the whole matrix; results are also compared across stages,
variants and tile sizes for bit identity (every kernel accumulates the k32
MFMA steps of an element in the same order; only a K split changes the
order, into per-piece sums added in piece order).
"""
import contextlib

import numpy as np
import pytest

import oracle
from software_pipelined_tiled_pipeline_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from software_pipelined_tiled_pipeline_amd import pgemm
    pgemm.lib()
    return pgemm


def dev_half(bits, fmt):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return t.view(torch.float16 if fmt == "f16" else torch.bfloat16)


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_nt(pg, fmt, variant, A, B, stages, dA=None, dB=None):
    dA = dev_half(A, fmt) if dA is None else dA
    dB = dev_half(B, fmt) if dB is None else dB
    name = f"pgemm_{fmt}_nt" + ("_ws" if variant == "ws" else "")
    out = getattr(pg, name)(dA, dB, stages=stages)
    torch.cuda.synchronize()
    return host_bits(out)


def assert_within_bound(fmt, got, ref, mag, what):
    bad, worst = oracle.check_nt(fmt, got, ref, mag)
    assert bad == 0, f"{what}: {bad} elements outside the bound (worst err/bound {worst:.3g})"
    return worst


VARIANTS = [("swap", 1), ("swap", 2), ("swap", 3), ("swap", 4), ("ws", 1), ("ws", 2), ("ws", 3), ("ws", 4)]
# (tile, k_split) forced through pgemm_set_tiling; (0, 0) is the planner's choice
TILINGS = [(256, 0), (128, 1), (128, 3)]


@contextlib.contextmanager
def tiling(pg, tile, split):
    pg.pgemm_set_tiling(tile, split)
    try:
        yield
    finally:
        pg.pgemm_set_tiling(0, 0)


# ------------------------------------------------------------------ int32

@pytest.mark.parametrize("stages", [1, 2])
def test_s32_workload_128x256x256(pg, stages):
    M, N, K = 128, 256, 256
    A, B = inputs.make_operands("s32_nn", M, N, K, inputs.workload_seed(1))
    out = pg.pgemm_s32_nn(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), stages=stages)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.gemm_s32_nn(A, B))


@pytest.mark.parametrize("M,N,K", [(37, 53, 29), (1, 1, 1), (16, 16, 16), (17, 15, 33), (200, 3, 0), (5, 300, 1)])
@pytest.mark.parametrize("stages", [1, 2])
def test_s32_ragged_and_wrapping(pg, M, N, K, stages):
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    A = rng.integers(-2 ** 31, 2 ** 31, (M, K)).astype(np.int32)
    B = rng.integers(-2 ** 31, 2 ** 31, (K, N)).astype(np.int32)
    out = pg.pgemm_s32_nn(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), stages=stages)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.gemm_s32_nn(A, B))


def s32_cases(n=16, seed=99):
    rng = np.random.default_rng(seed)
    return [(i, int(rng.integers(1, 700)), int(rng.integers(1, 700)), int(rng.integers(0, 300)), int(rng.integers(1, 3)))
            for i in range(n)]


@pytest.mark.parametrize("case", s32_cases(), ids=lambda c: "{}:{}x{}x{}-S{}".format(*c))
def test_s32_fuzzed_shapes(pg, case):
    # random shapes and full-range int32 operands, bit for bit
    i, M, N, K, stages = case
    rng = np.random.default_rng(1000 + i)
    A = rng.integers(-2 ** 31, 2 ** 31, (M, K)).astype(np.int32)
    B = rng.integers(-2 ** 31, 2 ** 31, (K, N)).astype(np.int32)
    out = pg.pgemm_s32_nn(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), stages=stages)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.gemm_s32_nn(A, B))


# ------------------------------------------------- NT, full comparisons

# K from one K tile up: at BK = 32 these give 7, 5, 1, 1, 2, 32, 3 and 4 K tiles
# (odd and even counts for the single schedule's two-tile loop body)
SMALL = [(520, 300, 200), (257, 129, 136), (64, 64, 8), (1, 1, 8), (300, 1000, 64), (513, 257, 1000), (96, 96, 96),
         (130, 70, 128)]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", SMALL)
def test_nt_small_all_variants(pg, fmt, M, N, K):
    kind = "f16_nt" if fmt == "f16" else "bf16_nt"
    A, B = inputs.make_operands(kind, M, N, K, 1000 + M + N + K)
    ref, mag = oracle.gemm_nt(fmt, A, B)
    dA, dB = dev_half(A, fmt), dev_half(B, fmt)
    unsplit = None
    for tile, split in TILINGS:
        with tiling(pg, tile, split):
            pieces = pg.pgemm_query("nt_ws", 0, M, N, K)["k_split"]
            first = None
            for variant, s in VARIANTS:
                got = run_nt(pg, fmt, variant, A, B, s, dA, dB)
                what = f"{fmt} {variant} S={s} tile {tile} pieces {pieces} {M}x{N}x{K}"
                assert_within_bound(fmt, got, ref, mag, what)
                if first is None:
                    first = got
                else:
                    assert np.array_equal(got, first), f"{what} differs in bits from swap S=1"
        if pieces == 1:  # tile size alone does not change an element's summation order
            if unsplit is None:
                unsplit = first
            else:
                assert np.array_equal(first, unsplit), f"tile {tile} differs in bits from tile 256"


def _random_shapes(seed, count):
    rng = np.random.default_rng(seed)
    shapes = []
    for _ in range(count):
        M = int(rng.integers(1, 521))
        N = int(rng.integers(1, 521))
        K = 8 * int(rng.integers(1, 129))  # rows of lhs/rhs start on 16 bytes
        shapes.append((M, N, K))
    return shapes


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", _random_shapes(2024, 6))
def test_nt_random_shapes_planned(pg, fmt, M, N, K):
    # seeded random shapes under the planner's own choice of tile and K
    # split (small shapes here take 128x128 tiles and often a split)
    kind = "f16_nt" if fmt == "f16" else "bf16_nt"
    A, B = inputs.make_operands(kind, M, N, K, 7000 + M + 3 * N + 5 * K)
    ref, mag = oracle.gemm_nt(fmt, A, B)
    dA, dB = dev_half(A, fmt), dev_half(B, fmt)
    q = pg.pgemm_query("nt_ws", 0, M, N, K)
    for variant, s in [("swap", 2), ("swap", 4), ("ws", 3)]:
        got = run_nt(pg, fmt, variant, A, B, s, dA, dB)
        assert_within_bound(fmt, got, ref, mag, f"{fmt} {variant} S={s} {M}x{N}x{K} pieces {q['k_split']}")


def fuzz_cases(n=48, seed=20261202):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        M = int(rng.choice([rng.integers(1, 40), rng.integers(100, 700), rng.integers(700, 1500)]))
        N = int(rng.choice([rng.integers(1, 40), rng.integers(100, 700), rng.integers(700, 1500)]))
        K = 8 * int(rng.choice([rng.integers(1, 8), rng.integers(8, 80), rng.integers(80, 260)]))
        fmt = str(rng.choice(["f16", "bf16"]))
        variant, stages = VARIANTS[int(rng.integers(len(VARIANTS)))]
        tile, split = [(0, 0), (128, 0), (128, 1), (128, 2), (128, 5), (256, 0), (256, 1)][int(rng.integers(7))]
        cases.append((i, M, N, K, fmt, variant, stages, tile, split))
    return cases


@pytest.mark.parametrize("case", fuzz_cases(), ids=lambda c: "{}:{}x{}x{}-{}-{}{}-t{}s{}".format(*c))
def test_nt_fuzzed_shapes_whole_output(pg, case):
    # random shapes (ragged edges, tiny and long K), formats, variants, stage
    # counts and forced tilings, each compared with the oracle in full
    i, M, N, K, fmt, variant, stages, tile, split = case
    kind = "f16_nt" if fmt == "f16" else "bf16_nt"
    A, B = inputs.make_operands(kind, M, N, K, 7000 + i)
    ref, mag = oracle.gemm_nt(fmt, A, B)
    with tiling(pg, tile, split):
        got = run_nt(pg, fmt, variant, A, B, stages)
    assert_within_bound(fmt, got, ref, mag, f"case {case}")


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("tile,split", TILINGS)
def test_nt_k_zero_gives_zeros(pg, fmt, tile, split):
    with tiling(pg, tile, split):
        _k_zero(pg, fmt)


def _k_zero(pg, fmt):
    for variant, s in VARIANTS:
        dA = torch.zeros((70, 0), dtype=torch.float16 if fmt == "f16" else torch.bfloat16, device="cuda")
        dB = torch.zeros((90, 0), dtype=dA.dtype, device="cuda")
        name = f"pgemm_{fmt}_nt" + ("_ws" if variant == "ws" else "")
        out = getattr(pg, name)(dA, dB, out=torch.full((70, 90), 7.0, dtype=dA.dtype, device="cuda"), stages=s)
        torch.cuda.synchronize()
        assert torch.count_nonzero(out).item() == 0


@pytest.mark.parametrize("tile,split", TILINGS)
@pytest.mark.parametrize("variant,stages", VARIANTS)
def test_nt_closed_forms(pg, variant, stages, tile, split):
    with tiling(pg, tile, split):
        _closed_forms(pg, variant, stages)


def _closed_forms(pg, variant, stages):
    # identity: lhs * I^T = lhs exactly
    K = 384
    A = inputs.f16_uniform1((300, K), 3, 0)
    I = np.where(np.eye(K, dtype=bool), np.uint16(0x3C00), np.uint16(0))
    assert np.array_equal(run_nt(pg, "f16", variant, A, I, stages), A)
    # all ones: exactly K (4096 is a binary16 value)
    ones_a = np.full((260, 4096), 0x3C00, np.uint16)
    ones_b = np.full((130, 4096), 0x3C00, np.uint16)
    got = run_nt(pg, "f16", variant, ones_a, ones_b, stages)
    assert np.all(got == np.float16(4096).view(np.uint16))
    # rank one: only k = 0 is non-zero, so out = RNE(u_m * v_n) with one rounding
    for fmt, kind in (("f16", "f16_nt"), ("bf16", "bf16_nt")):
        u, v = inputs.make_operands(kind, 270, 140, 8, 77)
        u[:, 1:] = 0
        v[:, 1:] = 0
        ref, _ = oracle.gemm_nt(fmt, u, v)
        assert np.array_equal(run_nt(pg, fmt, variant, u, v, stages), oracle.encode(fmt, ref))


# ------------------------------------------------------ tile boundaries

# Every K tail of both K tile depths (32 and 64) and of the element-guarded
# loader (K not a multiple of 8), n_k from 1 to 4 (fewer K tiles than the
# ring has slots at S = 3, 4), on output tiles cut one row or column short,
# exact, or one over.
BOUNDARY_K = [1, 7, 8, 24, 32, 33, 40, 56, 64, 65, 72, 96, 136, 200]


@pytest.mark.parametrize("tile", [128, 256])
@pytest.mark.parametrize("dm,dn", [(-1, -1), (-1, 0), (-1, 1), (0, -1), (0, 0), (0, 1), (1, -1), (1, 0), (1, 1)])
def test_nt_tile_boundaries(pg, tile, dm, dn):
    M, N = tile + dm, tile + dn
    for K in BOUNDARY_K:
        fmt = "f16" if K % 2 else "bf16"
        A, B = inputs.make_operands(f"{fmt}_nt", M, N, K, 4000 + 7 * K + dm + 3 * dn)
        ref, mag = oracle.gemm_nt(fmt, A, B)
        dA, dB = dev_half(A, fmt), dev_half(B, fmt)
        first = None
        with tiling(pg, tile, 1):
            for variant, s in VARIANTS:
                got = run_nt(pg, fmt, variant, A, B, s, dA, dB)
                what = f"{fmt} {variant} S={s} tile {tile} {M}x{N}x{K}"
                assert_within_bound(fmt, got, ref, mag, what)
                if first is None:
                    first = got
                else:
                    assert np.array_equal(got, first), f"{what} differs in bits from swap S=1"


# ----------------------------------------------------------- special values

# Several tiles with ragged edges on both tile sizes, and K = 203 (not a
# multiple of 8: the element-guarded staged loader).
SPECIAL_SHAPES = [(97, 83, 264), (300, 260, 1000), (65, 70, 203)]
SPECIAL_RUNS = [("swap", 2), ("swap", 4), ("ws", 3), ("ws", 4)]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("case", inputs.SPECIAL_CASES)
def test_nt_special_values(pg, fmt, case):
    # IEEE special values through every loader, schedule, tiling and K split
    # and the persistent schedule: NaN and infinities where the exact sum has
    # them, overflow to the infinity of the sum's sign, subnormal operands
    # (and binary32-subnormal sums for bfloat16) at their value, and sums of
    # zero products as +0
    for M, N, K in SPECIAL_SHAPES:
        A, B = inputs.special_operands(fmt, case, M, N, K, 900 + M + K)
        ref, mag = oracle.gemm_nt(fmt, A, B)
        dA, dB = dev_half(A, fmt), dev_half(B, fmt)
        outs = {}
        for tile, split in TILINGS + [(0, 0)]:
            with tiling(pg, tile, split):
                pieces = pg.pgemm_query("nt_ws", 0, M, N, K)["k_split"]
                first = None
                for variant, s in SPECIAL_RUNS:
                    got = run_nt(pg, fmt, variant, A, B, s, dA, dB)
                    what = f"{fmt} {case} {variant} S={s} tile {tile} pieces {pieces} {M}x{N}x{K}"
                    outs[what] = got
                    if first is None:
                        first = got
                    else:
                        assert np.array_equal(got, first), f"{what} differs in bits from {SPECIAL_RUNS[0]}"
        with tiling(pg, 128, 1), persistence(pg, 2):
            outs[f"{fmt} {case} persistent {M}x{N}x{K}"] = run_nt(pg, fmt, "ws", A, B, 4, dA, dB)
        for what, got in outs.items():
            assert_within_bound(fmt, got, ref, mag, what)
            if case == "zeros":
                assert np.all(got[np.arange(M) % 4 == 0] == 0), f"{what}: a zero lhs row gave a non-+0 bit pattern"
                assert np.all(got[:, np.arange(N) % 5 == 0] == 0), f"{what}: a -0 rhs row gave a non-+0 bit pattern"
    assert pg.pgemm_debug_status() == 0


# ------------------------------------------------------ full-size workloads

@pytest.fixture(scope="module")
def w2():
    return inputs.make_operands("f16_nt", 4096, 4096, 4096, inputs.workload_seed(2))


def check_whole(fmt, A, B, outs):
    """Every element of every output against the oracle."""
    ref, mag = oracle.gemm_nt(fmt, A, B)
    for what, got in outs.items():
        assert_within_bound(fmt, got, ref, mag, what)


def test_workload_f16_4096_swap2_vs_ws4(pg, w2):
    A, B = w2
    dA, dB = dev_half(A, "f16"), dev_half(B, "f16")
    outs = {
        "swap S=2": run_nt(pg, "f16", "swap", A, B, 2, dA, dB),
        "ws S=4": run_nt(pg, "f16", "ws", A, B, 4, dA, dB),
    }
    check_whole("f16", A, B, outs)
    assert np.array_equal(outs["swap S=2"], outs["ws S=4"])


def test_determinism_repeats(pg, w2):
    A, B = w2
    dA, dB = dev_half(A, "f16"), dev_half(B, "f16")
    first = run_nt(pg, "f16", "ws", A, B, 4, dA, dB)
    for _ in range(5):
        assert np.array_equal(run_nt(pg, "f16", "ws", A, B, 4, dA, dB), first)


def test_workload_f16_8192_stage_sweep(pg):
    A, B = inputs.make_operands("f16_nt", 8192, 8192, 8192, inputs.workload_seed(3))
    dA, dB = dev_half(A, "f16"), dev_half(B, "f16")
    outs = {f"ws S={s}": run_nt(pg, "f16", "ws", A, B, s, dA, dB) for s in (1, 2, 3, 4)}
    outs.update({f"swap S={s}": run_nt(pg, "f16", "swap", A, B, s, dA, dB) for s in (1, 2, 3, 4)})
    check_whole("f16", A, B, outs)
    first = outs["ws S=1"]
    for k, v in outs.items():
        assert np.array_equal(v, first), f"{k} differs in bits from ws S=1"


@pytest.fixture(scope="module")
def w4():
    M, N, K = 4095, 1000, 1000
    A, B = inputs.make_operands("bf16_nt", M, N, K, inputs.workload_seed(4))
    ref, mag = oracle.gemm_nt("bf16", A, B)
    return A, B, ref, mag


@pytest.mark.parametrize("tile", [0, 256])
@pytest.mark.parametrize("variant,stages", VARIANTS)
def test_workload_bf16_ragged_4095x1000x1000(pg, w4, variant, stages, tile):
    M, N, K = 4095, 1000, 1000
    A, B, ref, mag = w4
    with tiling(pg, tile, 0):
        got = run_nt(pg, "bf16", variant, A, B, stages)
        q = pg.pgemm_query("nt_ws" if variant == "ws" else "nt_swap", stages, M, N, K)
    assert q["block_m"] == (tile or 128)
    # report the edges separately: last partial row tile, last partial column tile
    em = (M // q["block_m"]) * q["block_m"]
    en = (N // q["block_n"]) * q["block_n"]
    assert_within_bound("bf16", got[em:], ref[em:], mag[em:], "partial M tile")
    assert_within_bound("bf16", got[:, en:], ref[:, en:], mag[:, en:], "partial N tile")
    assert_within_bound("bf16", got, ref, mag, f"bf16 {variant} S={stages}")


def test_workload_f16_skinny_128x8192x16384(pg):
    A, B = inputs.make_operands("f16_nt", 128, 8192, 16384, inputs.workload_seed(5))
    dA, dB = dev_half(A, "f16"), dev_half(B, "f16")
    assert pg.pgemm_query("nt_ws", 0, 128, 8192, 16384)["k_split"] == 4  # the planned split
    outs = {f"ws S={s}": run_nt(pg, "f16", "ws", A, B, s, dA, dB) for s in (1, 2, 3, 4)}
    outs.update({f"swap S={s}": run_nt(pg, "f16", "swap", A, B, s, dA, dB) for s in (1, 2, 3, 4)})
    with tiling(pg, 128, 1):
        unsplit = run_nt(pg, "f16", "ws", A, B, 4, dA, dB)
    with tiling(pg, 256, 0):
        large = run_nt(pg, "f16", "swap", A, B, 2, dA, dB)
    check_whole("f16", A, B, dict(outs, unsplit=unsplit, large=large))
    first = outs["ws S=1"]
    for k, v in outs.items():
        assert np.array_equal(v, first), k
    assert np.array_equal(unsplit, large)


def test_split_workspace_per_stream_and_growth(pg):
    # Two streams running K-split products at once each get their own
    # workspace; a larger split product on a stream grows that stream's.
    shapes = [(64, 1000, 4096, 2), (100, 700, 8192, 4), (128, 2000, 16384, 8)]
    data = []
    for i, (M, N, K, split) in enumerate(shapes):
        A, B = inputs.make_operands("f16_nt", M, N, K, 4242 + i)
        data.append((A, B, dev_half(A, "f16"), dev_half(B, "f16"), split))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = []
    for rep in range(2):
        for i, (A, B, dA, dB, split) in enumerate(data):
            with tiling(pg, 128, split):
                o = pg.pgemm_f16_nt_ws(dA, dB, stages=3, stream=streams[(i + rep) % 2])
                o2 = pg.pgemm_f16_nt(dA, dB, stages=2, stream=streams[(i + rep + 1) % 2])
                outs.append((i, o, o2))
    torch.cuda.synchronize()
    results = {}
    for i, o, o2 in outs:
        got, got2 = host_bits(o), host_bits(o2)
        assert np.array_equal(got, got2)
        if i in results:
            assert np.array_equal(got, results[i])
        results[i] = got
    for i, (A, B, _, _, split) in enumerate(data):
        ref, mag = oracle.gemm_nt("f16", A, B)
        assert_within_bound("f16", results[i], ref, mag, f"split {split}")


# --------------------------------------------------- persistent schedule

@contextlib.contextmanager
def persistence(pg, mode):
    pg.pgemm_set_persistent(mode)
    try:
        yield
    finally:
        pg.pgemm_set_persistent(0)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("tile,M,N,K", [(128, 2560, 2048, 136), (128, 2600, 2050, 72), (256, 4608, 4352, 264),
                                        (256, 4100, 4500, 8), (128, 300, 200, 64)])
def test_persistent_matches_per_tile_kernel(pg, fmt, tile, M, N, K):
    # more tiles than the persistent grid holds, so workgroups stride over
    # several tiles (ragged edges in the last ones); same bits as the
    # per-tile kernel, and inside the bound on every element
    kind = "f16_nt" if fmt == "f16" else "bf16_nt"
    A, B = inputs.make_operands(kind, M, N, K, 31 + M + K)
    dA, dB = dev_half(A, fmt), dev_half(B, fmt)
    with tiling(pg, tile, 1):
        for S in (1, 2, 3, 4):
            with persistence(pg, 2):
                q = pg.pgemm_query("nt_ws", S, M, N, K)
                assert q["persistent"] == 1
                got = run_nt(pg, fmt, "ws", A, B, S, dA, dB)
            with persistence(pg, 1):
                ref_bits = run_nt(pg, fmt, "ws", A, B, S, dA, dB)
            assert np.array_equal(got, ref_bits), f"persistent S={S} differs from the per-tile kernel"
    check_whole(fmt, A, B, {"persistent": got})
    assert pg.pgemm_debug_status() == 0


def persistent_cases(n=16, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        tile = int(rng.choice([128, 256]))
        M = int(rng.integers(1, 5 * tile * 8))
        N = int(rng.integers(1, 5 * tile * 4))
        K = 8 * int(rng.integers(1, 100))
        out.append((i, tile, M, N, K, str(rng.choice(["f16", "bf16"])), int(rng.integers(1, 5))))
    return out


@pytest.mark.parametrize("case", persistent_cases(), ids=lambda c: "{}:t{}-{}x{}x{}-{}-S{}".format(*c))
def test_persistent_fuzzed_against_per_tile_kernel(pg, case):
    # random shapes on both tile sizes: the persistent schedule gives the
    # per-tile kernel's bits
    i, tile, M, N, K, fmt, S = case
    kind = "f16_nt" if fmt == "f16" else "bf16_nt"
    A, B = inputs.make_operands(kind, M, N, K, 8000 + i)
    dA, dB = dev_half(A, fmt), dev_half(B, fmt)
    with tiling(pg, tile, 1):
        with persistence(pg, 2):
            got = run_nt(pg, fmt, "ws", A, B, S, dA, dB)
        with persistence(pg, 1):
            want = run_nt(pg, fmt, "ws", A, B, S, dA, dB)
    assert np.array_equal(got, want)
    assert pg.pgemm_debug_status() == 0


def test_persistent_k_zero(pg):
    dA = torch.zeros((700, 0), dtype=torch.float16, device="cuda")
    dB = torch.zeros((900, 0), dtype=torch.float16, device="cuda")
    with tiling(pg, 128, 1), persistence(pg, 2):
        out = pg.pgemm_f16_nt_ws(dA, dB, out=torch.full((700, 900), 3.0, dtype=torch.float16, device="cuda"))
        torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


# ------------------------------------------------ concurrent streams

def test_many_small_gemms_on_concurrent_streams(pg):
    # independent products on four streams at once (Croqtile ch.5,
    # parallel.async with a stream per grid): each call only enqueues, the
    # grids may overlap on the device, and every result must be the one a
    # lone call gives (the K-split ones use their stream's own workspace)
    shapes = [(256, 384, 512), (300, 200, 1000), (128, 1024, 4096), (520, 260, 136), (64, 2048, 2048),
              (1000, 130, 64), (128, 512, 8192), (384, 384, 384)]
    cases = []
    for i, (M, N, K) in enumerate(shapes):
        A, B = inputs.make_operands("f16_nt", M, N, K, 900 + i)
        cases.append((A, B, dev_half(A, "f16"), dev_half(B, "f16")))
    alone = []
    for i, (A, B, dA, dB) in enumerate(cases):
        alone.append(run_nt(pg, "f16", "ws" if i % 2 else "swap", A, B, 2 + i % 3, dA, dB))
    streams = [torch.cuda.Stream() for _ in range(4)]
    torch.cuda.synchronize()
    outs = []
    for rep in range(3):
        for i, (A, B, dA, dB) in enumerate(cases):
            f = pg.pgemm_f16_nt_ws if i % 2 else pg.pgemm_f16_nt
            outs.append((i, f(dA, dB, stages=2 + i % 3, stream=streams[(i + rep) % 4])))
    torch.cuda.synchronize()
    for i, o in outs:
        assert np.array_equal(host_bits(o), alone[i]), f"case {i} differs when run concurrently"
    for i, (A, B, _, _) in enumerate(cases):
        ref, mag = oracle.gemm_nt("f16", A, B)
        assert_within_bound("f16", alone[i], ref, mag, f"case {i}")


# ----------------------------------------------------- credit protocol

def test_missing_seed_times_out_instead_of_hanging(pg):
    # Without the consumers' initial empty credits the producers' first wait
    # can never succeed.  With a small poll limit every wait gives up, the
    # kernel still exits, and the host sees PGEMM_ERR_TIMEOUT.
    A, B = inputs.make_operands("f16_nt", 256, 128, 128, 9)
    dA, dB = dev_half(A, "f16"), dev_half(B, "f16")
    assert pg.pgemm_debug_status() == 0
    try:
        pg.pgemm_set_ws_debug(max_polls=2000, skip_seed=True)
        pg.pgemm_f16_nt_ws(dA, dB, stages=2)
        assert pg.pgemm_debug_status() == 7  # PGEMM_ERR_TIMEOUT
    finally:
        pg.pgemm_set_ws_debug(0, False)
    assert pg.pgemm_debug_status() == 0
    got = run_nt(pg, "f16", "ws", A, B, 2, dA, dB)
    ref, mag = oracle.gemm_nt("f16", A, B)
    assert_within_bound("f16", got, ref, mag, "after reset")
    assert pg.pgemm_debug_status() == 0
    # the persistent kernel's waits are bounded the same way
    with tiling(pg, 128, 1), persistence(pg, 2):
        try:
            pg.pgemm_set_ws_debug(max_polls=2000, skip_seed=True)
            pg.pgemm_f16_nt_ws(dA, dB, stages=2)
            assert pg.pgemm_debug_status() == 7
        finally:
            pg.pgemm_set_ws_debug(0, False)
        assert pg.pgemm_debug_status() == 0
        got = run_nt(pg, "f16", "ws", A, B, 2, dA, dB)
    assert_within_bound("f16", got, ref, mag, "persistent, after reset")


@contextlib.contextmanager
def credit_jitter(pg, seed):
    pg.pgemm_set_ws_jitter(seed)
    try:
        yield
    finally:
        pg.pgemm_set_ws_jitter(0)


# (tile, k_split, persistent mode, M, N, K): every producer/consumer code
# path -- whole tiles per producer (32-deep slots) and tiles shared by all
# producers (64-deep), consumers with one and with two fragment sets, a K
# split, and the persistent schedule on both tile sizes
JITTER_CASES = [(256, 1, 0, 700, 600, 520), (128, 1, 0, 700, 650, 1000), (128, 3, 0, 300, 260, 1000),
                (256, 1, 2, 1100, 1030, 264), (128, 1, 2, 700, 650, 200)]


@pytest.mark.parametrize("case", JITTER_CASES, ids=lambda c: "t{}s{}p{}-{}x{}x{}".format(*c))
def test_ws_credit_jitter_keeps_bits(pg, case):
    # Random sleeps before every credit wait and trigger make producers and
    # consumers meet in other orders than their natural timing gives; every
    # stage count must still give the same bits, and no wait may give up.
    tile, split, persist, M, N, K = case
    fmt = "bf16" if tile == 128 else "f16"
    A, B = inputs.make_operands(f"{fmt}_nt", M, N, K, 600 + M + K)
    dA, dB = dev_half(A, fmt), dev_half(B, fmt)
    assert pg.pgemm_debug_status() == 0
    with tiling(pg, tile, split), persistence(pg, persist):
        for S in (1, 2, 3, 4):
            want = run_nt(pg, fmt, "ws", A, B, S, dA, dB)
            for seed in (1, 0x5A5A5, 0x7FFFFFFF):
                with credit_jitter(pg, seed):
                    got = run_nt(pg, fmt, "ws", A, B, S, dA, dB)
                assert np.array_equal(got, want), f"S={S} jitter seed {seed:#x} changed the bits"
            assert pg.pgemm_debug_status() == 0
    check_whole(fmt, A, B, {"jittered": got})


# ------------------------------------------- single schedule, split barriers

@pytest.mark.gpu
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(520, 300, 4160), (257, 511, 8200), (300, 260, 64 * 41 + 40), (256, 256, 128)])
def test_split_barrier_schedule_long_and_ragged_k(pg, fmt, M, N, K):
    """The 256 x 256 single schedule at S = 2 (separate WAR and RAW barriers
    per K tile): long K with an odd and an even number of K tiles, a K tail
    inside the last tile, ragged M and N, compared with the oracle element
    by element, and bit-identical to S = 1 (same k order, one barrier)."""
    A, B = inputs.make_operands(fmt + "_nt", M, N, K, 700 + M + K)
    ref, mag = oracle.gemm_nt(fmt, A, B)
    dA, dB = dev_half(A, fmt), dev_half(B, fmt)
    with tiling(pg, 256, 0):
        assert pg.pgemm_query("nt_swap", 2, M, N, K)["block_m"] == 256
        got = run_nt(pg, fmt, "swap", A, B, 2, dA, dB)
        one = run_nt(pg, fmt, "swap", A, B, 1, dA, dB)
    assert_within_bound(fmt, got, ref, mag, f"{fmt} {M}x{N}x{K} swap S=2, 256 x 256")
    assert np.array_equal(got, one), "S = 2 and S = 1 differ"
