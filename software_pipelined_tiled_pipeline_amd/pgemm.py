"""Python binding of the pgemm C-ABI (argument marshalling only).

Each function takes torch tensors that already live on the current GPU,
passes their device pointers and the current HIP stream to the library
function of the same name, and raises ``PgemmError`` on a non-zero status.
All arithmetic runs in the library's HIP kernels; there is no other path:
if ``libpgemm.so`` has not been built, every call raises.

The library never allocates.  For a product the planner splits along K, the
NT functions here first make sure the stream has a registered fp32
workspace of the planned size: a torch tensor allocated on that stream and
handed to ``pgemm_set_workspace`` (torch is the device-memory provider).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpgemm.so")

STATUS = {
    0: "PGEMM_OK", 1: "PGEMM_ERR_NULL", 2: "PGEMM_ERR_SHAPE", 3: "PGEMM_ERR_STAGES",
    4: "PGEMM_ERR_ALIGN", 5: "PGEMM_ERR_LDS", 6: "PGEMM_ERR_LAUNCH", 7: "PGEMM_ERR_TIMEOUT",
    8: "PGEMM_ERR_DEVICE", 9: "PGEMM_ERR_WORKSPACE",
}
OPS = {"s32_nn": 0, "nt_swap": 1, "nt_ws": 2}
GEMM_SYMBOLS = ("pgemm_s32_nn", "pgemm_f16_nt", "pgemm_f16_nt_ws", "pgemm_bf16_nt", "pgemm_bf16_nt_ws",
                "pgemm_f16_nt_ws_static")


class PgemmError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({strerror(status)})")


class KernelInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "block_m", "block_n", "block_k", "stages", "producer_waves", "consumer_waves", "threads", "lds_bytes")] + [
        ("grid", ctypes.c_int64), ("k_tiles", ctypes.c_int64), ("k_split", ctypes.c_int32),
        ("persistent", ctypes.c_int32), ("workspace_bytes", ctypes.c_int64), ("staged", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        for name in GEMM_SYMBOLS:
            f = getattr(L, name)
            f.argtypes = [P, P, P, I64, I64, I64, I, P]
            f.restype = I
        L.pgemm_query.argtypes = [I, I, I64, I64, I64, ctypes.POINTER(KernelInfo)]
        L.pgemm_query.restype = I
        L.pgemm_debug_status.argtypes = [P]
        L.pgemm_debug_status.restype = I
        L.pgemm_set_workspace.argtypes = [P, P, I64]
        L.pgemm_set_workspace.restype = I
        L.pgemm_set_tiling.argtypes = [I, I]
        L.pgemm_set_tiling.restype = I
        L.pgemm_set_persistent.argtypes = [I]
        L.pgemm_set_persistent.restype = I
        L.pgemm_set_ws_debug.argtypes = [I64, I]
        L.pgemm_set_ws_debug.restype = None
        L.pgemm_set_ws_jitter.argtypes = [ctypes.c_uint32]
        L.pgemm_set_ws_jitter.restype = None
        L.pgemm_strerror.argtypes = [I]
        L.pgemm_strerror.restype = ctypes.c_char_p
        L.pgemm_abi_version.argtypes = []
        L.pgemm_abi_version.restype = I
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().pgemm_strerror(status).decode()


def abi_version() -> int:
    return lib().pgemm_abi_version()


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, what: str):
    if status != 0:
        raise PgemmError(status, what)


def _call(name, lhs, rhs, out, M, N, K, stages, stream):
    f = getattr(lib(), name)
    _check(f(lhs.data_ptr() or None, rhs.data_ptr() or None, out.data_ptr() or None,
             M, N, K, int(stages), _stream(stream)), name)
    return out


def _operands(lhs, rhs, out, dtype, nn: bool):
    import torch
    if not torch.cuda.is_available():
        raise ValueError("pgemm needs a GPU")
    here = torch.device("cuda", torch.cuda.current_device())
    for t in (lhs, rhs):
        if t.dtype != dtype or t.dim() != 2 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"operands must be contiguous 2-D {dtype} CUDA tensors")
        if t.device != here:
            raise ValueError(f"operands must be on the current device {here}, not {t.device}")
    M, K = lhs.shape
    if nn:
        K2, N = rhs.shape
    else:
        N, K2 = rhs.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if out is None:
        out = torch.empty((M, N), dtype=dtype, device=here)
    elif out.dtype != dtype or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, N] tensor of the operand type")
    elif not out.is_cuda or out.device != here:
        raise ValueError(f"out must be on the current device {here}")
    return out, M, N, K


# (device index, stream handle) -> the uint8 tensor registered as that
# stream's K-split workspace
_workspaces = {}


def ensure_workspace(nbytes: int, stream=None):
    """Registers a workspace of at least `nbytes` for `stream` (default: the
    current stream) on the current device, growing the registered one if it
    is smaller; returns the tensor.  It is allocated on that stream, so that
    torch reuses a replaced buffer only for later work on the same stream."""
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    key = (torch.cuda.current_device(), s.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(s):
            ws = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device="cuda")
        _check(lib().pgemm_set_workspace(ctypes.c_void_p(s.cuda_stream), ctypes.c_void_p(ws.data_ptr()),
                                         ws.numel()), "pgemm_set_workspace")
        _workspaces[key] = ws
    return ws


def release_workspace(stream=None) -> None:
    """Unregisters the workspace of `stream` (after the work that used it)."""
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    key = (torch.cuda.current_device(), s.cuda_stream)
    _check(lib().pgemm_set_workspace(ctypes.c_void_p(s.cuda_stream), None, 0), "pgemm_set_workspace")
    _workspaces.pop(key, None)


def pgemm_s32_nn(lhs, rhs, out=None, stages: int = 0, stream=None):
    """int32 out[M,N] = lhs[M,K] @ rhs[K,N] (wrapping), swap double buffering."""
    import torch
    out, M, N, K = _operands(lhs, rhs, out, torch.int32, nn=True)
    return _call("pgemm_s32_nn", lhs, rhs, out, M, N, K, stages, stream)


def _nt(name, dtype_name):
    op = "nt_ws" if name.endswith("_ws") else "nt_swap"

    def fn(lhs, rhs, out=None, stages: int = 0, stream=None, split: bool = True):
        import torch
        out, M, N, K = _operands(lhs, rhs, out, getattr(torch, dtype_name), nn=False)
        if split and M and N:
            need = pgemm_query(op, stages, M, N, K)["workspace_bytes"]
            if need:
                ensure_workspace(need, stream)
        return _call(name, lhs, rhs, out, M, N, K, stages, stream)
    fn.__name__ = name
    fn.__doc__ = (f"{dtype_name} out[M,N] = lhs[M,K] @ rhs[N,K]^T with fp32 accumulation (library call {name}); "
                  "split=False leaves the stream's workspace as it is (a call without one runs unsplit).")
    return fn


pgemm_f16_nt = _nt("pgemm_f16_nt", "float16")
pgemm_f16_nt_ws = _nt("pgemm_f16_nt_ws", "float16")


def pgemm_f16_nt_ws_static(lhs, rhs, out=None, stages: int = 0, stream=None):
    """pgemm_f16_nt_ws whose K-split partial sums live in the library's static
    per-device scratch: the library allocates nothing (library call of the
    same name).  Calls that may overlap on one device race on that scratch."""
    import torch
    out, M, N, K = _operands(lhs, rhs, out, torch.float16, nn=False)
    return _call("pgemm_f16_nt_ws_static", lhs, rhs, out, M, N, K, stages, stream)


pgemm_bf16_nt = _nt("pgemm_bf16_nt", "bfloat16")
pgemm_bf16_nt_ws = _nt("pgemm_bf16_nt_ws", "bfloat16")


def pgemm_query(op: str, stages: int, M: int, N: int, K: int) -> dict:
    info = KernelInfo()
    _check(lib().pgemm_query(OPS[op], stages, M, N, K, ctypes.byref(info)), "pgemm_query")
    return {n: getattr(info, n) for n, _ in KernelInfo._fields_}


def pgemm_debug_status(stream=None) -> int:
    return lib().pgemm_debug_status(_stream(stream))


def pgemm_set_tiling(tile: int = 0, k_split: int = 0) -> None:
    """Forces the tiling of later NT calls (0, 0 restores the planner)."""
    _check(lib().pgemm_set_tiling(int(tile), int(k_split)), "pgemm_set_tiling")


def pgemm_set_persistent(mode: int = 0) -> None:
    """Producer/consumer schedule of later calls: 0 planned, 1 never, 2 always persistent."""
    _check(lib().pgemm_set_persistent(int(mode)), "pgemm_set_persistent")


def pgemm_set_ws_debug(max_polls: int = 0, skip_seed: bool = False) -> None:
    lib().pgemm_set_ws_debug(int(max_polls), 1 if skip_seed else 0)


def pgemm_set_ws_jitter(seed: int = 0) -> None:
    """Credit-timing jitter of later producer/consumer calls (0: off)."""
    lib().pgemm_set_ws_jitter(int(seed) & 0x7FFFFFFF)
