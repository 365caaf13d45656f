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


# Special-value operands (the edge cases of IEEE 754 half-precision input):
#
# * "subnormal": rows in three classes by index mod 3, in both operands.
#   binary16: 0 = every element subnormal (exponent field 0, fraction 1..1023,
#   random sign), 1 = the uniform recipe, 2 = each element subnormal or
#   uniform with probability 1/2.  bfloat16: 0 = every element subnormal
#   (fraction 1..127), 1 = the normal recipe, 2 = the normal recipe times
#   2**50 (so that subnormal x class 2 products are normal binary32 values,
#   and no sum leaves binary32's range).
# * "overflow": binary16: the uniform recipe times 2**7 (sums over a few
#   hundred k reach past 65504 in both directions); bfloat16: magnitudes of
#   the normal recipe times 2**(58 + m mod 6) for lhs row m and 2**62 for
#   every rhs row, lhs rows of odd m negated (every product of an element
#   has one sign, so sums grow monotonically past the largest finite value).
# * "nonfinite": the standard recipe with infinities and NaNs planted at
#   fixed positions (edges of the K range and of the matrices included) and
#   a zero facing one of the infinities (see ``_plant_nonfinite``).
# * "zeros": the standard recipe with lhs rows of m mod 4 == 0 set to zeros of
#   random sign and rhs rows of n mod 5 == 0 set to -0.
SPECIAL_CASES = ("subnormal", "overflow", "nonfinite", "zeros")
_SPECIAL = {
    "f16": {"inf": 0x7C00, "ninf": 0xFC00, "nan": 0x7E00, "frac": 0x3FF, "exp_shift": 10},
    "bf16": {"inf": 0x7F80, "ninf": 0xFF80, "nan": 0x7FC0, "frac": 0x7F, "exp_shift": 7},
}


def _subnormal_bits(fmt, shape, seed, tensor):
    n = int(np.prod(shape))
    x = splitmix64(tensor_key(seed, tensor), 0, n)
    frac = np.uint64(_SPECIAL[fmt]["frac"])
    mag = (x % frac + np.uint64(1)).astype(np.uint16)
    sign = ((x >> np.uint64(63)).astype(np.uint16) << np.uint16(15))
    return (mag | sign).reshape(shape)


def _scale_exponent(fmt, bits, add):
    """bits times 2**add for normal, nonzero values (exponent field + add)."""
    bits = np.asarray(bits, np.uint16)
    shift = _SPECIAL[fmt]["exp_shift"]
    exp = (bits.astype(np.int64) >> shift) & (0x1F if fmt == "f16" else 0xFF)
    add = np.broadcast_to(np.asarray(add, np.int64), bits.shape)
    top = 0x1F if fmt == "f16" else 0xFF
    if np.any((exp > 0) & (exp + add >= top)):
        raise ValueError("scaled value leaves the normal range")
    return np.where(exp > 0, bits.astype(np.int64) + (add << shift), bits).astype(np.uint16)


def _plant_nonfinite(fmt, A, B):
    s = _SPECIAL[fmt]
    M, K = A.shape
    N = B.shape[0]
    A, B = A.copy(), B.copy()
    k5 = min(5, K - 1)
    A[1 % M, k5] = s["inf"]
    A[2 % M, K - 1] = s["ninf"]
    A[3 % M, 0] = s["nan"]
    if K >= 2:
        A[4 % M, K // 2] = s["inf"]
        A[4 % M, K // 2 - 1] = s["ninf"]
    A[M - 1, 0] = s["inf"]
    B[2 % N, k5] = 0            # faces the infinity of lhs row 1
    B[5 % N, K // 3] = s["inf"]
    B[6 % N, K - 1] = s["nan"]
    B[N - 1, K - 1] = s["ninf"]
    return A, B


def special_operands(fmt: str, case: str, M: int, N: int, K: int, seed: int):
    """(lhs[M,K], rhs[N,K]) half-precision bits for one special-value case."""
    if fmt not in _SPECIAL or case not in SPECIAL_CASES:
        raise ValueError(f"unknown special case {fmt!r} {case!r}")
    A, B = make_operands(f"{fmt}_nt", M, N, K, seed)
    if case == "subnormal":
        def classes(X, tensor):
            sub = _subnormal_bits(fmt, X.shape, seed, 2 + tensor)
            cls = (np.arange(X.shape[0]) % 3)[:, None]
            if fmt == "f16":
                coin = (splitmix64(tensor_key(seed, 4 + tensor), 0, X.size) & np.uint64(1)).reshape(X.shape) == 1
                return np.where(cls == 0, sub, np.where((cls == 2) & coin, sub, X)).astype(np.uint16)
            return np.where(cls == 0, sub, np.where(cls == 2, _scale_exponent(fmt, X, 50), X)).astype(np.uint16)
        return classes(A, 0), classes(B, 1)
    if case == "overflow":
        if fmt == "f16":
            scale = lambda X: (X.view(np.float16).astype(np.float32) * 128.0).astype(np.float16).view(np.uint16)
            return scale(A), scale(B)
        m = np.arange(M)[:, None]
        A = _scale_exponent(fmt, A & np.uint16(0x7FFF), 58 + m % 6) | np.where(m % 2 == 1, 0x8000, 0).astype(np.uint16)
        B = _scale_exponent(fmt, B & np.uint16(0x7FFF), 62)
        return A.astype(np.uint16), B.astype(np.uint16)
    if case == "nonfinite":
        return _plant_nonfinite(fmt, A, B)
    zero_sign = ((splitmix64(tensor_key(seed, 6), 0, A.size) & np.uint64(1)).astype(np.uint16) << np.uint16(15))
    A = np.where((np.arange(M) % 4 == 0)[:, None], zero_sign.reshape(A.shape), A).astype(np.uint16)
    B = np.where((np.arange(N) % 5 == 0)[:, None], np.uint16(0x8000), B).astype(np.uint16)
    return A, B
