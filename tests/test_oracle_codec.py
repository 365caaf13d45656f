"""Pins for the oracle's half-precision codecs and ulp function.

Each check sets the oracle's own IEEE-754 code against an independent
implementation: numpy's binary16 (decode, RNE encode, spacing), numpy's
binary32 bit view (bfloat16 decode), and torch's float32 -> bfloat16
conversion (round-to-nearest-even).
"""
import numpy as np
import pytest
import torch

import oracle


def _same(a, b):
    return np.all((a == b) | (np.isnan(a) & np.isnan(b)))


def test_f16_decode_all_patterns():
    h = np.arange(65536, dtype=np.uint16)
    assert _same(oracle.decode("f16", h), h.view(np.float16).astype(np.float64))


def test_bf16_decode_all_patterns():
    h = np.arange(65536, dtype=np.uint16)
    as_f32 = (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert _same(oracle.decode("bf16", h), as_f32)


def _f16_probe_values(rng):
    e = rng.integers(-30, 18, size=200000)
    v = rng.random(200000) * 2.0 ** e.astype(np.float64) * rng.choice([-1.0, 1.0], 200000)
    # exact ties between neighbours, across the subnormal and normal range
    h = rng.integers(0, 0x7BFF, size=20000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    ties = (lo + hi) / 2.0
    edges = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e30, -1e30,
                      2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26,
                      2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11,
                      1.0 + 3 * 2.0 ** -11, np.inf, -np.inf, np.nan])
    return np.concatenate([v, ties, -ties, edges])


def test_f16_encode_matches_numpy():
    v = _f16_probe_values(np.random.default_rng(1))
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16)
    got = oracle.encode("f16", v).view(np.float16)
    assert _same(got.astype(np.float64), ref.astype(np.float64))
    # signs of zeros too
    z = np.array([0.0, -0.0, -2.0 ** -30])
    assert list(oracle.encode("f16", z)) == [0x0000, 0x8000, 0x8000]


def test_bf16_encode_matches_torch():
    rng = np.random.default_rng(2)
    e = rng.integers(-140, 128, size=200000)
    v32 = (rng.random(200000) * 2.0 ** e.astype(np.float64)).astype(np.float32)
    v32 = v32 * rng.choice([-1.0, 1.0], 200000).astype(np.float32)
    # binary32 values exactly halfway between two bfloat16 neighbours
    hb = rng.integers(0, 0x7F7F, size=20000).astype(np.uint32)
    ties = ((hb << 16) | 0x8000).view(np.float32)
    v32 = np.concatenate([v32, ties, -ties, np.array([0.0, 3.3895314e38], np.float32)])
    ref = torch.from_numpy(v32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.encode("bf16", v32.astype(np.float64))
    assert np.array_equal(got, ref)
    assert list(oracle.encode("bf16", np.array([np.inf, -np.inf, 2.0 ** 128]))) == [0x7F80, 0xFF80, 0x7F80]


def test_ulp_f16_matches_numpy_spacing():
    h = np.arange(0, 0x7C00, dtype=np.uint16)  # all finite non-negative values
    y = h.view(np.float16)
    ref = np.spacing(y).astype(np.float64)
    # spacing of the largest finite value is inf in numpy; the ulp of its binade is 32
    ref[-1] = 32.0
    assert np.array_equal(oracle.ulp("f16", y.astype(np.float64)), ref)
    assert np.array_equal(oracle.ulp("f16", -y.astype(np.float64)), ref)


def test_ulp_bf16_closed_form():
    # bfloat16 keeps 7 fraction bits: its spacing is 2**16 times binary32's
    # for normal values, and 2**-133 below 2**-126.
    h = np.arange(0x0080, 0x7F7F, 7, dtype=np.uint32)
    y = (h << 16).view(np.float32)
    ref = np.spacing(y).astype(np.float64) * 2.0 ** 16
    assert np.array_equal(oracle.ulp("bf16", y.astype(np.float64)), ref)
    assert oracle.ulp("bf16", np.array([0.0, 2.0 ** -127]))[0] == 2.0 ** -133
    assert oracle.ulp("bf16", np.array([1.0]))[0] == 2.0 ** -7
    assert oracle.ulp("f16", np.array([1.0, 0.0, 2.0 ** -15]))[0] == 2.0 ** -10
