"""CPU oracle for the tiled GEMMs (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library neither imports nor links it, and it
shares no code with the GPU library: the arithmetic lives in ``oracle.c``
(plain C, OpenMP over output rows, built with ``-ffp-contract=off``), and this
module only marshals numpy arrays into it.

What it computes is the plain matrix product (see the header of ``oracle.c``
for the passages followed and the readings taken):

* ``gemm_s32_nn(lhs[M,K], rhs[K,N])`` -> int32 ``[M,N]``, sums modulo 2**32.
* ``gemm_nt(fmt, lhs[M,K], rhs[N,K])`` -> (``ref``, ``mag``) float64 ``[M,N]``:
  ``ref = sum_k a*b`` in k order in binary64, ``mag = sum_k |a*b|``.
* ``check_nt`` applies the acceptance bound
  ``|g - ref| <= rel*mag + ulp(RNE(ref))`` in the output format; a NaN or
  infinite ``ref`` must come out as NaN or as the same infinity, and an
  infinite output is accepted for a finite ``ref`` of its sign that lies
  within the bound of the format's overflow threshold or beyond it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F16 = 0
BF16 = 1
FORMATS = {"f16": F16, "bf16": BF16}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm",
        ])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.pgo_decode.argtypes = [ctypes.c_int, P, P, I64]
        lib.pgo_encode.argtypes = [ctypes.c_int, P, P, I64]
        lib.pgo_ulp.argtypes = [ctypes.c_int, P, P, I64]
        lib.pgo_gemm_s32_nn.argtypes = [P, P, P, I64, I64, I64]
        lib.pgo_gemm_nt.argtypes = [ctypes.c_int, P, P, P, P, I64, I64, I64]
        lib.pgo_gemm_nt.restype = ctypes.c_int
        lib.pgo_gemm_nt_entries.argtypes = [ctypes.c_int, P, P, I64, I64, I64, P, P, I64, P, P]
        lib.pgo_gemm_nt_entries.restype = ctypes.c_int
        lib.pgo_check_nt.argtypes = [ctypes.c_int, P, P, P, I64, ctypes.c_double,
                                     ctypes.POINTER(ctypes.c_double)]
        lib.pgo_check_nt.restype = ctypes.c_int64
        lib.pgo_threads.argtypes = []
        lib.pgo_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().pgo_threads())


def _fmt(fmt) -> int:
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def decode(fmt, bits) -> np.ndarray:
    bits, p = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float64)
    _load().pgo_decode(_fmt(fmt), p, out.ctypes.data, bits.size)
    return out


def encode(fmt, values) -> np.ndarray:
    values, p = _c(values, np.float64)
    out = np.empty(values.shape, np.uint16)
    _load().pgo_encode(_fmt(fmt), p, out.ctypes.data, values.size)
    return out


def ulp(fmt, values) -> np.ndarray:
    values, p = _c(values, np.float64)
    out = np.empty(values.shape, np.float64)
    _load().pgo_ulp(_fmt(fmt), p, out.ctypes.data, values.size)
    return out


def gemm_s32_nn(lhs, rhs) -> np.ndarray:
    lhs, pa = _c(lhs, np.int32)
    rhs, pb = _c(rhs, np.int32)
    M, K = lhs.shape
    K2, N = rhs.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    out = np.empty((M, N), np.int32)
    _load().pgo_gemm_s32_nn(pa, pb, out.ctypes.data, M, N, K)
    return out


def gemm_nt(fmt, lhs, rhs):
    lhs, pa = _c(lhs, np.uint16)
    rhs, pb = _c(rhs, np.uint16)
    M, K = lhs.shape
    N, K2 = rhs.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    ref = np.empty((M, N), np.float64)
    mag = np.empty((M, N), np.float64)
    if _load().pgo_gemm_nt(_fmt(fmt), pa, pb, ref.ctypes.data, mag.ctypes.data, M, N, K):
        raise MemoryError("oracle decode table")
    return ref, mag


def gemm_nt_entries(fmt, lhs, rhs, mi, ni):
    lhs, pa = _c(lhs, np.uint16)
    rhs, pb = _c(rhs, np.uint16)
    M, K = lhs.shape
    N, K2 = rhs.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    mi, pm = _c(mi, np.int64)
    ni, pn = _c(ni, np.int64)
    if mi.shape != ni.shape:
        raise ValueError("index arrays differ in shape")
    if mi.size and (mi.min() < 0 or mi.max() >= M or ni.min() < 0 or ni.max() >= N):
        raise IndexError("entry index out of range")
    ref = np.empty(mi.shape, np.float64)
    mag = np.empty(mi.shape, np.float64)
    if _load().pgo_gemm_nt_entries(_fmt(fmt), pa, pb, M, N, K, pm, pn, mi.size,
                                   ref.ctypes.data, mag.ctypes.data):
        raise MemoryError("oracle decode table")
    return ref, mag


def check_nt(fmt, got, ref, mag, rel: float = 1e-3):
    """Return (number of elements outside the bound, worst |err|/bound)."""
    got, pg = _c(got, np.uint16)
    ref, pr = _c(ref, np.float64)
    mag, pm = _c(mag, np.float64)
    if not (got.shape == ref.shape == mag.shape):
        raise ValueError("shape mismatch")
    worst = ctypes.c_double(0.0)
    bad = _load().pgo_check_nt(_fmt(fmt), pg, pr, pm, got.size, rel, ctypes.byref(worst))
    return int(bad), float(worst.value)
