"""ctypes binding of libmoda (include/moda.h): argument marshalling only.

The functions named like the C entry points (``moda_fwd``, ``moda_bwd``, ...)
take torch tensors that the caller allocated, pass their device pointers and
the current HIP stream, and raise ``ModaError`` on a non-OK status.  ``fwd``,
``bwd`` and ``pack_depth`` additionally allocate the outputs with torch.  Every
step of the computation runs in the HIP kernels of libmoda.so; there is no
fallback: if the library is missing this module raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoda.so")

MODA_OK, MODA_ERR_INVALID_ARGUMENT, MODA_ERR_UNSUPPORTED, MODA_ERR_HIP = 0, 1, 2, 3
MODA_BF16, MODA_F32 = 0, 1
MODA_MAX_L = 1024

EXPORTS = ("moda_fwd", "moda_bwd", "moda_bwd_workspace_bytes", "moda_pack_depth",
           "moda_status_string", "moda_last_error", "moda_fwd_chunk_tokens", "moda_timing_arm",
           "moda_timing_count", "moda_timing_label")


class ModaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Hk", ctypes.c_int64),
                ("T", ctypes.c_int64), ("d", ctypes.c_int64), ("L", ctypes.c_int64),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libmoda.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"libmoda.so not found at {path}: run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        P, I = ctypes.c_void_p, ctypes.c_int
        PP = ctypes.POINTER(Problem)
        lib.moda_fwd.argtypes = [PP] + [P] * 8
        lib.moda_fwd.restype = I
        lib.moda_bwd.argtypes = [PP] + [P] * 14 + [ctypes.c_size_t, P]
        lib.moda_bwd.restype = I
        lib.moda_bwd_workspace_bytes.argtypes = [PP]
        lib.moda_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.moda_pack_depth.argtypes = [PP, P, P, P]
        lib.moda_pack_depth.restype = I
        lib.moda_status_string.argtypes = [I]
        lib.moda_status_string.restype = ctypes.c_char_p
        lib.moda_last_error.argtypes = []
        lib.moda_last_error.restype = ctypes.c_char_p
        lib.moda_fwd_chunk_tokens.argtypes = [PP]
        lib.moda_fwd_chunk_tokens.restype = ctypes.c_int32
        lib.moda_timing_arm.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32]
        lib.moda_timing_arm.restype = I
        lib.moda_timing_count.argtypes = []
        lib.moda_timing_count.restype = ctypes.c_int32
        lib.moda_timing_label.argtypes = [ctypes.c_int32]
        lib.moda_timing_label.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def problem(B, Hq, Hk, T, d, L, scale=None, dtype=MODA_BF16, chunk=0, reserved=0) -> Problem:
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return Problem(B, Hq, Hk, T, d, L, scale, dtype, chunk, reserved)


def problem_for(Q: torch.Tensor, K: torch.Tensor, L: int, scale=None, chunk=0) -> Problem:
    B, Hq, T, d = Q.shape
    dt = {torch.bfloat16: MODA_BF16, torch.float32: MODA_F32}.get(Q.dtype)
    if dt is None:
        raise TypeError(f"unsupported dtype {Q.dtype}")
    return problem(B, Hq, K.shape[1], T, d, L, scale, dt, chunk)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(rc: int):
    if rc != MODA_OK:
        lib = load()
        raise ModaError(rc, f"{lib.moda_status_string(rc).decode()}: "
                            f"{lib.moda_last_error().decode()}")


def moda_fwd(p: Problem, Q, K, V, Kd, Vd, O, lse, stream=None) -> None:
    _check(load().moda_fwd(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(Kd), _ptr(Vd),
                           _ptr(O), _ptr(lse), _stream(stream)))


def moda_bwd_workspace_bytes(p: Problem) -> int:
    return int(load().moda_bwd_workspace_bytes(ctypes.byref(p)))


def moda_bwd(p: Problem, Q, K, V, Kd, Vd, O, lse, dO, dQ, dK, dV, dKd, dVd, workspace,
             workspace_bytes=None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(load().moda_bwd(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(Kd), _ptr(Vd),
                           _ptr(O), _ptr(lse), _ptr(dO), _ptr(dQ), _ptr(dK), _ptr(dV),
                           _ptr(dKd), _ptr(dVd), _ptr(workspace), int(workspace_bytes),
                           _stream(stream)))


def moda_pack_depth(p: Problem, layers, packed, stream=None) -> None:
    _check(load().moda_pack_depth(ctypes.byref(p), _ptr(layers), _ptr(packed), _stream(stream)))


def moda_fwd_chunk_tokens(p: Problem) -> int:
    return int(load().moda_fwd_chunk_tokens(ctypes.byref(p)))


class KernelTimer:
    """Per-kernel HIP-event timing through moda_timing_arm.

    Creates `capacity` hipEvent_t handles with the HIP runtime, arms libmoda
    with them, and after a synchronisation returns (label, milliseconds) for
    every kernel libmoda launched on this thread since arming."""

    def __init__(self, capacity: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = (ctypes.c_void_p * capacity)()
        for i in range(capacity):
            ev = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.events[i] = ev.value
        self.capacity = capacity

    def arm(self):
        _check(load().moda_timing_arm(self.events, self.capacity))

    def disarm(self):
        _check(load().moda_timing_arm(None, 0))

    def results(self):
        lib = load()
        out = []
        for i in range(lib.moda_timing_count()):
            a, b = self.events[2 * i], self.events[2 * i + 1]
            if self.hip.hipEventSynchronize(b) != 0:
                raise RuntimeError("hipEventSynchronize failed")
            ms = ctypes.c_float()
            if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append((lib.moda_timing_label(i).decode(), ms.value))
        return out

    def close(self):
        for e in self.events:
            if e:
                self.hip.hipEventDestroy(e)
        self.events = None


# ---- allocating conveniences (torch allocates; libmoda computes) ----

def fwd(Q, K, V, Kd, Vd, L, scale=None, chunk=0, stream=None):
    """O [B,Hq,T,d] (dtype of Q) and lse [B,Hq,T] fp32."""
    p = problem_for(Q, K, L, scale, chunk)
    O = torch.empty_like(Q)
    lse = torch.empty(Q.shape[:3], device=Q.device, dtype=torch.float32)
    moda_fwd(p, Q, K, V, Kd, Vd, O, lse, stream)
    return O, lse


def bwd(Q, K, V, Kd, Vd, O, lse, dO, L, scale=None, chunk=0, stream=None):
    """(dQ, dK, dV, dKd, dVd); dKd/dVd are None when L == 0."""
    p = problem_for(Q, K, L, scale, chunk)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    dKd = torch.empty_like(Kd) if L > 0 else None
    dVd = torch.empty_like(Vd) if L > 0 else None
    ws = torch.empty(max(moda_bwd_workspace_bytes(p), 256), device=Q.device, dtype=torch.uint8)
    moda_bwd(p, Q, K, V, Kd, Vd, O, lse, dO, dQ, dK, dV, dKd, dVd, ws, stream=stream)
    return dQ, dK, dV, dKd, dVd


def pack_depth(layers, stream=None):
    """layers [L,B,Hk,T,d] -> packed [B,Hk,T*L,d]."""
    L, B, Hk, T, d = layers.shape
    dt = {torch.bfloat16: MODA_BF16, torch.float32: MODA_F32}[layers.dtype]
    p = problem(B, Hk, Hk, T, d, L, 1.0, dt)
    out = torch.empty((B, Hk, T * L, d), device=layers.device, dtype=layers.dtype)
    moda_pack_depth(p, layers, out, stream)
    return out
