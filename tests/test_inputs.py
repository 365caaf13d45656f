"""The seeded operand generator: published SplitMix64 outputs, determinism,
and the value ranges of each workload's recipe."""
import numpy as np

from software_pipelined_tiled_pipeline_amd import inputs


def test_splitmix64_published_outputs():
    # The first outputs of SplitMix64 from state 0, as published with the
    # generator (Steele, Lea & Flood 2014; also java.util.SplittableRandom).
    got = [int(v) for v in inputs.splitmix64(0, 0, 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_based_chunks_agree():
    whole = inputs.splitmix64(12345, 0, 10000)
    parts = np.concatenate([inputs.splitmix64(12345, s, 1000) for s in range(0, 10000, 1000)])
    assert np.array_equal(whole, parts)


def test_recipes():
    s = inputs.workload_seed(1)
    A = inputs.int32_uniform8((128, 256), s, 0)
    assert A.dtype == np.int32 and A.min() == -8 and A.max() == 8
    assert set(np.unique(A)) == set(range(-8, 9))
    assert np.array_equal(A, inputs.int32_uniform8((128, 256), s, 0))
    assert not np.array_equal(A, inputs.int32_uniform8((128, 256), s, 1))
    h = inputs.f16_uniform1((300, 700), 3, 0).view(np.float16).astype(np.float64)
    assert h.min() >= -1.0 and h.max() <= 1.0 and abs(h.mean()) < 0.01
    b = inputs.bf16_normal((400, 1000), 4, 0)
    v = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1.0) < 0.01


def test_bf16_rounding_is_ties_to_even():
    import torch
    rng = np.random.default_rng(0)
    x32 = rng.standard_normal(100000).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(inputs.f64_to_bf16_bits(x32.astype(np.float64)), ref)


def _decode(fmt, bits):
    bits = np.asarray(bits, np.uint16)
    if fmt == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_special_recipes():
    M, N, K = 31, 29, 40
    for fmt, tiny in (("f16", 2.0 ** -14), ("bf16", 2.0 ** -126)):
        base = inputs.make_operands(f"{fmt}_nt", M, N, K, 9)
        # subnormal: class 0 rows all subnormal, class 1 rows the plain recipe
        A, B = inputs.special_operands(fmt, "subnormal", M, N, K, 9)
        for X, X0 in ((A, base[0]), (B, base[1])):
            v = _decode(fmt, X)
            assert np.all((np.abs(v[0::3]) < tiny) & (v[0::3] != 0))
            assert np.array_equal(X[1::3], X0[1::3])
            if fmt == "f16":   # class 2 mixes the two, element by element
                sub = (np.abs(v[2::3]) < tiny) & (v[2::3] != 0)
                assert 0.3 < sub.mean() < 0.7
                assert np.array_equal(X[2::3][~sub], X0[2::3][~sub])
            else:              # class 2 is the plain recipe times 2**50, exactly
                assert np.array_equal(v[2::3], _decode(fmt, X0[2::3]) * 2.0 ** 50)
        # overflow: exact power-of-two scalings
        A, B = inputs.special_operands(fmt, "overflow", M, N, K, 9)
        if fmt == "f16":
            assert np.array_equal(_decode(fmt, A), _decode(fmt, base[0]) * 128)
            assert np.array_equal(_decode(fmt, B), _decode(fmt, base[1]) * 128)
        else:
            m = np.arange(M)[:, None]
            want = np.abs(_decode(fmt, base[0])) * 2.0 ** (58 + m % 6) * np.where(m % 2 == 1, -1.0, 1.0)
            assert np.array_equal(_decode(fmt, A), want)
            assert np.array_equal(_decode(fmt, B), np.abs(_decode(fmt, base[1])) * 2.0 ** 62)
        # nonfinite: the plain recipe except at the planted positions
        A, B = inputs.special_operands(fmt, "nonfinite", M, N, K, 9)
        va, vb = _decode(fmt, A), _decode(fmt, B)
        assert np.isinf(va[1, 5]) and va[1, 5] > 0 and va[2, K - 1] == -np.inf and np.isnan(va[3, 0])
        assert va[4, K // 2] == np.inf and va[4, K // 2 - 1] == -np.inf and va[M - 1, 0] == np.inf
        assert vb[2, 5] == 0 and vb[5, K // 3] == np.inf and np.isnan(vb[6, K - 1]) and vb[N - 1, K - 1] == -np.inf
        assert np.sum(A != base[0]) <= 6 and np.sum(B != base[1]) <= 4
        # zeros: lhs rows m % 4 == 0 are zeros of both signs, rhs rows n % 5 == 0 are -0
        A, B = inputs.special_operands(fmt, "zeros", M, N, K, 9)
        assert np.all((A[0::4] & 0x7FFF) == 0) and 0 < np.mean(A[0::4] == 0x8000) < 1
        assert np.all(B[0::5] == 0x8000)
        assert np.array_equal(A[1::4], base[0][1::4]) and np.array_equal(B[1::5], base[1][1::5])
