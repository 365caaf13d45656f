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
