"""Seeded synthetic operands for the GEMM workloads.

This module only draws numbers: it holds no matrix arithmetic, so both the
CPU oracle's checks and the GPU path can take their operands from here.

Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), used counter-based.  Element ``i`` of a
tensor keyed ``key`` is the ``i``-th output of a SplitMix64 stream whose state
starts at ``key``:

    z = key + (i + 1) * 0x9E3779B97F4A7C15          (mod 2**64)
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9
    z = (z ^ (z >> 27)) * 0x94D049BB133111EB
    x = z ^ (z >> 31)

so a value never depends on how many threads or chunks produced it.
``key = seed ^ (tensor << 56)``.

Distributions (the workloads' recipes):

* ``int32`` "uniform in [-8, 8]": ``(x mod 17) - 8`` (integers -8..8).
* ``f16`` "uniform in [-1, 1]": ``u = (x >> 11) * 2**-53`` in [0, 1),
  value ``2u - 1`` rounded to binary16 with ties-to-even.
* ``bf16`` "normal(0, 1)": Box-Muller on two uniforms
  (``u1 = ((x0 >> 11) + 1) * 2**-53`` in (0, 1], ``u2 = (x1 >> 11) * 2**-53``),
  ``sqrt(-2 ln u1) * cos(2 pi u2)``, rounded to bfloat16 with ties-to-even.

Half-precision results are returned as ``uint16`` bit patterns.
"""
from __future__ import annotations

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def splitmix64(key: int, start: int, count: int) -> np.ndarray:
    """Outputs ``start .. start+count-1`` of the SplitMix64 stream seeded ``key``."""
    key = np.uint64(key & 0xFFFFFFFFFFFFFFFF)
    out = np.empty(count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        for lo in range(0, count, _CHUNK):
            n = min(_CHUNK, count - lo)
            z = np.arange(start + lo + 1, start + lo + 1 + n, dtype=np.uint64)
            z *= _GAMMA
            z += key
            z ^= z >> np.uint64(30)
            z *= _M1
            z ^= z >> np.uint64(27)
            z *= _M2
            z ^= z >> np.uint64(31)
            out[lo:lo + n] = z
    return out


def tensor_key(seed: int, tensor: int) -> int:
    return (seed ^ (tensor << 56)) & 0xFFFFFFFFFFFFFFFF


def _unit(x: np.ndarray) -> np.ndarray:
    return (x >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def int32_uniform8(shape, seed: int, tensor: int) -> np.ndarray:
    """Integers uniform in -8..8 (inclusive), int32, row-major ``shape``."""
    n = int(np.prod(shape))
    x = splitmix64(tensor_key(seed, tensor), 0, n)
    return ((x % np.uint64(17)).astype(np.int64) - 8).astype(np.int32).reshape(shape)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round binary64 values to bfloat16 (ties-to-even) and return the bits.

    Exact for finite inputs whose magnitude lies in bfloat16's normal range or
    is zero; these are the only values the generators produce.
    """
    v = np.asarray(v, dtype=np.float64)
    bits = v.view(np.uint64)
    sign = (bits >> np.uint64(63)).astype(np.uint32)
    exp = ((bits >> np.uint64(52)) & np.uint64(0x7FF)).astype(np.int64)
    mant = bits & np.uint64((1 << 52) - 1)
    nz = exp != 0
    if np.any(nz & ((exp - 1023 < -126) | (exp - 1023 > 127))):
        raise ValueError("value outside bfloat16 normal range")
    # keep 7 of the 52 fraction bits, ties to even on the 45 dropped bits
    keep = mant >> np.uint64(45)
    rest = mant & np.uint64((1 << 45) - 1)
    half = np.uint64(1 << 44)
    up = (rest > half) | ((rest == half) & ((keep & np.uint64(1)) == 1))
    mag = ((exp - 1023 + 127).astype(np.uint64) << np.uint64(7)) + keep + up.astype(np.uint64)
    mag = np.where(nz, mag, np.uint64(0)).astype(np.uint32)
    return ((sign << np.uint32(15)) | mag).astype(np.uint16)


def f16_uniform1(shape, seed: int, tensor: int) -> np.ndarray:
    """binary16 bits of values uniform in [-1, 1)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    key = tensor_key(seed, tensor)
    for lo in range(0, n, _CHUNK):
        m = min(_CHUNK, n - lo)
        u = _unit(splitmix64(key, lo, m))
        out[lo:lo + m] = (2.0 * u - 1.0).astype(np.float16).view(np.uint16)
    return out.reshape(shape)


def bf16_normal(shape, seed: int, tensor: int) -> np.ndarray:
    """bfloat16 bits of standard normal values (Box-Muller, cosine branch)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    key = tensor_key(seed, tensor)
    for lo in range(0, n, _CHUNK):
        m = min(_CHUNK, n - lo)
        x = splitmix64(key, 2 * lo, 2 * m)
        u1 = ((x[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)
        u2 = _unit(x[1::2])
        z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
        z = np.where(np.abs(z) < 2.0 ** -126, 0.0, z)
        out[lo:lo + m] = f64_to_bf16_bits(z)
    return out.reshape(shape)


# Seeds: 0x5EED0000 + 16 * workload + tensor index (0 = lhs, 1 = rhs).
SEED_BASE = 0x5EED0000


def workload_seed(workload: int) -> int:
    return SEED_BASE + 16 * workload


def make_operands(kind: str, M: int, N: int, K: int, seed: int):
    """Return (lhs, rhs) for one GEMM.

    kind "s32_nn": lhs int32[M,K], rhs int32[K,N], values -8..8.
    kind "f16_nt": lhs f16[M,K], rhs f16[N,K], uniform [-1, 1).
    kind "bf16_nt": lhs bf16[M,K], rhs bf16[N,K], normal(0, 1).
    """
    if kind == "s32_nn":
        return int32_uniform8((M, K), seed, 0), int32_uniform8((K, N), seed, 1)
    if kind == "f16_nt":
        return f16_uniform1((M, K), seed, 0), f16_uniform1((N, K), seed, 1)
    if kind == "bf16_nt":
        return bf16_normal((M, K), seed, 0), bf16_normal((N, K), seed, 1)
    raise ValueError(f"unknown operand kind {kind!r}")
