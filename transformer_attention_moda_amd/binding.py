"""ctypes binding of libmoda (include/moda.h): argument marshalling only.

The functions named like the C entry points (``moda_fwd``, ``moda_bwd``, ...)
take torch tensors that the caller allocated, check that each one is a
contiguous GPU tensor of the shape and dtype the problem implies (the C ABI
takes bare pointers and cannot), pass their device pointers and the current
HIP stream, and raise ``ModaError`` on a non-OK status.  A plain int is taken
as a raw device pointer and passed through unchecked.  ``fwd``, ``bwd`` and
``pack_depth`` additionally allocate the outputs with torch.  Every step of the
computation runs in the HIP kernels of libmoda.so; there is no fallback: if the
library is missing this module raises.
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
MODA_NONCAUSAL = 1
MODA_NOALLOC_SCRATCH_BYTES = 256 << 20
MODA_SCAN_WAVE, MODA_SCAN_CHUNK, MODA_SCAN_ALL = 0, 1, 2
_TORCH_DTYPE = {MODA_BF16: torch.bfloat16, MODA_F32: torch.float32}

EXPORTS = ("moda_fwd", "moda_bwd", "moda_bwd_workspace_bytes", "moda_bwd_noalloc",
           "moda_decode", "moda_decode_workspace_bytes", "moda_depth_append", "moda_pack_depth",
           "moda_fwd_depth_scan",
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
                ("flags", ctypes.c_int32), ("window", ctypes.c_int32), ("reserved", ctypes.c_int32)]


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
        lib.moda_bwd_noalloc.argtypes = [PP] + [P] * 14
        lib.moda_bwd_noalloc.restype = I
        lib.moda_bwd_workspace_bytes.argtypes = [PP]
        lib.moda_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.moda_decode_workspace_bytes.argtypes = [PP]
        lib.moda_decode_workspace_bytes.restype = ctypes.c_size_t
        lib.moda_decode.argtypes = [PP, ctypes.c_int64] + [P] * 8 + [ctypes.c_size_t, P]
        lib.moda_decode.restype = I
        lib.moda_depth_append.argtypes = [PP, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          P, P]
        lib.moda_depth_append.restype = I
        lib.moda_fwd_depth_scan.argtypes = [PP, ctypes.c_int32] + [P] * 8
        lib.moda_fwd_depth_scan.restype = I
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


def problem(B, Hq, Hk, T, d, L, scale=None, dtype=MODA_BF16, chunk=0, flags=0, window=0,
            reserved=0) -> Problem:
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return Problem(B, Hq, Hk, T, d, L, scale, dtype, chunk, flags, window, reserved)


def problem_for(Q: torch.Tensor, K: torch.Tensor, L: int, scale=None, chunk=0, causal=True,
                window=0) -> Problem:
    if Q.dim() != 4 or K.dim() != 4:
        raise ValueError(f"Q and K must be 4-D [B,H,T,d]; got {tuple(Q.shape)}, {tuple(K.shape)}")
    B, Hq, T, d = Q.shape
    dt = {torch.bfloat16: MODA_BF16, torch.float32: MODA_F32}.get(Q.dtype)
    if dt is None:
        raise TypeError(f"unsupported dtype {Q.dtype}")
    return problem(B, Hq, K.shape[1], T, d, L, scale, dt, chunk,
                   0 if causal else MODA_NONCAUSAL, window)


def _structure(name, t, shape, dtype, optional=False):
    """Raise unless t is a contiguous tensor of this shape and dtype.  An int is a raw
    device pointer, passed unchecked; None is allowed only when optional."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if isinstance(t, int):
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor or a raw device pointer")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}; the problem needs {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}; the problem needs {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} is not contiguous (a transposed or strided view?)")


def _check_tensors(specs):
    """specs: (name, tensor, shape, dtype[, optional]).  First every tensor's shape,
    dtype and layout, then that all of them sit on one GPU."""
    for spec in specs:
        _structure(*spec)
    dev = None
    for name, t, *_ in specs:
        if not isinstance(t, torch.Tensor):
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} is on {t.device}, not on a GPU")
        if dev is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}; the other tensors are on {dev}")
        dev = t.device


def _workspace_bytes(workspace, workspace_bytes):
    """Usable bytes of a workspace tensor (never more than it holds), or the given count
    for a raw pointer."""
    if isinstance(workspace, torch.Tensor):
        if not workspace.is_contiguous() or workspace.device.type != "cuda":
            raise ValueError("workspace must be a contiguous GPU tensor")
        nbytes = workspace.numel() * workspace.element_size()
        return nbytes if workspace_bytes is None else min(int(workspace_bytes), nbytes)
    if workspace_bytes is None:
        raise ValueError("workspace_bytes is required with a raw workspace pointer")
    return int(workspace_bytes)


def _shapes(p: Problem):
    q = (p.B, p.Hq, p.T, p.d)
    kv = (p.B, p.Hk, p.T, p.d)
    dep = (p.B, p.Hk, p.T * p.L, p.d)
    return q, kv, dep, (p.B, p.Hq, p.T)


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
    dt = _TORCH_DTYPE.get(p.dtype)
    if dt is not None:
        q, kv, dep, rows = _shapes(p)
        nodep = p.L == 0
        _check_tensors([("Q", Q, q, dt), ("K", K, kv, dt), ("V", V, kv, dt),
                        ("Kd", Kd, dep, dt, nodep), ("Vd", Vd, dep, dt, nodep),
                        ("O", O, q, dt), ("lse", lse, rows, torch.float32)])
    _check(load().moda_fwd(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(Kd), _ptr(Vd),
                           _ptr(O), _ptr(lse), _stream(stream)))


def moda_fwd_depth_scan(p: Problem, scan: int, Q, K, V, Kd, Vd, O, lse, stream=None) -> None:
    """The forward with another depth-row scan (MODA_SCAN_*), for the layout ablation."""
    dt = _TORCH_DTYPE.get(p.dtype)
    if dt is not None:
        q, kv, dep, rows = _shapes(p)
        nodep = p.L == 0
        _check_tensors([("Q", Q, q, dt), ("K", K, kv, dt), ("V", V, kv, dt),
                        ("Kd", Kd, dep, dt, nodep), ("Vd", Vd, dep, dt, nodep),
                        ("O", O, q, dt), ("lse", lse, rows, torch.float32)])
    _check(load().moda_fwd_depth_scan(ctypes.byref(p), int(scan), _ptr(Q), _ptr(K), _ptr(V),
                                      _ptr(Kd), _ptr(Vd), _ptr(O), _ptr(lse), _stream(stream)))


def moda_bwd_workspace_bytes(p: Problem) -> int:
    return int(load().moda_bwd_workspace_bytes(ctypes.byref(p)))


def moda_bwd(p: Problem, Q, K, V, Kd, Vd, O, lse, dO, dQ, dK, dV, dKd, dVd, workspace,
             workspace_bytes=None, stream=None) -> None:
    dt = _TORCH_DTYPE.get(p.dtype)
    if dt is not None:
        q, kv, dep, rows = _shapes(p)
        nodep = p.L == 0
        _check_tensors([("Q", Q, q, dt), ("K", K, kv, dt), ("V", V, kv, dt),
                        ("Kd", Kd, dep, dt, nodep), ("Vd", Vd, dep, dt, nodep),
                        ("O", O, q, dt), ("lse", lse, rows, torch.float32), ("dO", dO, q, dt),
                        ("dQ", dQ, q, dt), ("dK", dK, kv, dt), ("dV", dV, kv, dt),
                        ("dKd", dKd, dep, dt, nodep), ("dVd", dVd, dep, dt, nodep)])
    workspace_bytes = _workspace_bytes(workspace, workspace_bytes)
    _check(load().moda_bwd(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(Kd), _ptr(Vd),
                           _ptr(O), _ptr(lse), _ptr(dO), _ptr(dQ), _ptr(dK), _ptr(dV),
                           _ptr(dKd), _ptr(dVd), _ptr(workspace), int(workspace_bytes),
                           _stream(stream)))


def moda_bwd_noalloc(p: Problem, Q, K, V, Kd, Vd, O, lse, dO, dQ, dK, dV, dKd, dVd,
                     stream=None) -> None:
    """moda_bwd with the library's static per-GPU scratch instead of a workspace (for
    callers that cannot allocate); calls that overlap on one GPU race."""
    dt = _TORCH_DTYPE.get(p.dtype)
    if dt is not None:
        q, kv, dep, rows = _shapes(p)
        nodep = p.L == 0
        _check_tensors([("Q", Q, q, dt), ("K", K, kv, dt), ("V", V, kv, dt),
                        ("Kd", Kd, dep, dt, nodep), ("Vd", Vd, dep, dt, nodep),
                        ("O", O, q, dt), ("lse", lse, rows, torch.float32), ("dO", dO, q, dt),
                        ("dQ", dQ, q, dt), ("dK", dK, kv, dt), ("dV", dV, kv, dt),
                        ("dKd", dKd, dep, dt, nodep), ("dVd", dVd, dep, dt, nodep)])
    _check(load().moda_bwd_noalloc(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(Kd),
                                   _ptr(Vd), _ptr(O), _ptr(lse), _ptr(dO), _ptr(dQ), _ptr(dK),
                                   _ptr(dV), _ptr(dKd), _ptr(dVd), _stream(stream)))


def moda_pack_depth(p: Problem, layers, packed, stream=None) -> None:
    dt = _TORCH_DTYPE.get(p.dtype)
    if dt is not None:
        _check_tensors([("layers", layers, (p.L, p.B, p.Hk, p.T, p.d), dt),
                        ("packed", packed, (p.B, p.Hk, p.T * p.L, p.d), dt)])
    _check(load().moda_pack_depth(ctypes.byref(p), _ptr(layers), _ptr(packed), _stream(stream)))


def moda_decode_workspace_bytes(p: Problem) -> int:
    return int(load().moda_decode_workspace_bytes(ctypes.byref(p)))


def moda_decode(p: Problem, pos: int, q, K, V, Kd, Vd, O, lse, workspace, workspace_bytes=None,
                stream=None) -> None:
    """One new query token at cache position pos: q, O [B,Hq,d]; lse [B,Hq]; K, V
    [B,Hk,T,d] and Kd, Vd [B,Hk,T*L,d] caches of T tokens."""
    dt = _TORCH_DTYPE.get(p.dtype)
    if dt is not None:
        _, kv, dep, _ = _shapes(p)
        nodep = p.L == 0
        _check_tensors([("q", q, (p.B, p.Hq, p.d), dt), ("K", K, kv, dt), ("V", V, kv, dt),
                        ("Kd", Kd, dep, dt, nodep), ("Vd", Vd, dep, dt, nodep),
                        ("O", O, (p.B, p.Hq, p.d), dt), ("lse", lse, (p.B, p.Hq), torch.float32)])
    workspace_bytes = _workspace_bytes(workspace, workspace_bytes)
    _check(load().moda_decode(ctypes.byref(p), int(pos), _ptr(q), _ptr(K), _ptr(V), _ptr(Kd),
                              _ptr(Vd), _ptr(O), _ptr(lse), _ptr(workspace), int(workspace_bytes),
                              _stream(stream)))


def moda_depth_append(p: Problem, layer, slot: int, t0: int, packed, stream=None) -> None:
    """Write layer [B,Hk,n,d] (tokens t0..t0+n-1) into slot `slot` of packed [B,Hk,T*L,d]."""
    dt = _TORCH_DTYPE.get(p.dtype)
    n = layer.shape[2] if isinstance(layer, torch.Tensor) and layer.dim() == 4 else None
    if n is None:
        raise ValueError("layer must be a [B,Hk,n,d] tensor")
    if dt is not None:
        _check_tensors([("layer", layer, (p.B, p.Hk, n, p.d), dt),
                        ("packed", packed, (p.B, p.Hk, p.T * p.L, p.d), dt)])
    _check(load().moda_depth_append(ctypes.byref(p), _ptr(layer), int(slot), int(t0), int(n),
                                    _ptr(packed), _stream(stream)))


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
            label = lib.moda_timing_label(i)
            out.append((label.decode() if label else "?", ms.value))
        return out

    def close(self):
        for e in self.events:
            if e:
                self.hip.hipEventDestroy(e)
        self.events = None


# ---- allocating conveniences (torch allocates; libmoda computes) ----

def fwd(Q, K, V, Kd, Vd, L, scale=None, chunk=0, stream=None, causal=True, window=0):
    """O [B,Hq,T,d] (dtype of Q) and lse [B,Hq,T] fp32."""
    p = problem_for(Q, K, L, scale, chunk, causal, window)
    O = torch.empty_like(Q)
    lse = torch.empty(Q.shape[:3], device=Q.device, dtype=torch.float32)
    moda_fwd(p, Q, K, V, Kd, Vd, O, lse, stream)
    return O, lse


def bwd(Q, K, V, Kd, Vd, O, lse, dO, L, scale=None, chunk=0, stream=None, causal=True,
        window=0):
    """(dQ, dK, dV, dKd, dVd); dKd/dVd are None when L == 0."""
    p = problem_for(Q, K, L, scale, chunk, causal, window)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    dKd = torch.empty_like(Kd) if L > 0 else None
    dVd = torch.empty_like(Vd) if L > 0 else None
    ws = torch.empty(max(moda_bwd_workspace_bytes(p), 256), device=Q.device, dtype=torch.uint8)
    moda_bwd(p, Q, K, V, Kd, Vd, O, lse, dO, dQ, dK, dV, dKd, dVd, ws, stream=stream)
    return dQ, dK, dV, dKd, dVd


def pack_depth(layers, stream=None):
    """layers [L,B,Hk,T,d] -> packed [B,Hk,T*L,d]."""
    if layers.dim() != 5:
        raise ValueError(f"layers must be [L,B,Hk,T,d]; got shape {tuple(layers.shape)}")
    L, B, Hk, T, d = layers.shape
    dt = {torch.bfloat16: MODA_BF16, torch.float32: MODA_F32}.get(layers.dtype)
    if dt is None:
        raise TypeError(f"unsupported dtype {layers.dtype}")
    p = problem(B, Hk, Hk, T, d, L, 1.0, dt)
    out = torch.empty((B, Hk, T * L, d), device=layers.device, dtype=layers.dtype)
    moda_pack_depth(p, layers, out, stream)
    return out


def decode(q, K, V, Kd, Vd, L, pos, scale=None, window=0, causal=True, stream=None):
    """(O [B,Hq,d], lse [B,Hq]) of one new token at cache position pos."""
    B, Hq, d = q.shape
    Hk, T = K.shape[1], K.shape[2]
    dt = {torch.bfloat16: MODA_BF16, torch.float32: MODA_F32}.get(q.dtype)
    if dt is None:
        raise TypeError(f"unsupported dtype {q.dtype}")
    p = problem(B, Hq, Hk, T, d, L, scale, dt, 0, 0 if causal else MODA_NONCAUSAL, window)
    O = torch.empty_like(q)
    lse = torch.empty((B, Hq), device=q.device, dtype=torch.float32)
    ws = torch.empty(max(moda_decode_workspace_bytes(p), 256), device=q.device,
                     dtype=torch.uint8)
    moda_decode(p, pos, q, K, V, Kd, Vd, O, lse, ws, stream=stream)
    return O, lse


def depth_append(packed, layer, L, slot, t0=0, stream=None):
    """Write layer [B,Hk,n,d] into slot `slot` of packed [B,Hk,T*L,d] in place."""
    B, Hk, TL, d = packed.shape
    if TL % L:
        raise ValueError("packed rows are not a multiple of L")
    dt = {torch.bfloat16: MODA_BF16, torch.float32: MODA_F32}.get(packed.dtype)
    if dt is None:
        raise TypeError(f"unsupported dtype {packed.dtype}")
    p = problem(B, Hk, Hk, TL // L, d, L, 1.0, dt)
    moda_depth_append(p, layer, slot, t0, packed, stream)
    return packed


class DepthKVCache:
    """The depth rows of L slots per token for one attention call, as the packed pair
    Kd, Vd [B,Hk,T*L,d] (token-major: row t*L + slot) that moda_fwd, moda_bwd and
    moda_decode read, filled one layer at a time by moda_depth_append.  This is the role the
    moda-attention 0.1.0 PyPI page ("Architecture") gives its DepthKVCache: contiguous depth
    KV storage across layers.  The tensors start as zeros; a caller writes every slot it lets
    the operator see before calling it."""

    def __init__(self, B, Hk, T, L, d, dtype=torch.bfloat16, device="cuda"):
        if min(B, Hk, T, L, d) < 1:
            raise ValueError(f"B, Hk, T, L and d must be >= 1; got {(B, Hk, T, L, d)}")
        self.L = int(L)
        self.K = torch.zeros((B, Hk, T * L, d), dtype=dtype, device=device)
        self.V = torch.zeros_like(self.K)

    def append(self, k_layer, v_layer, slot, t0=0, stream=None):
        """Write one layer's K and V rows [B,Hk,n,d] of tokens t0..t0+n-1 into depth slot
        `slot` of both tensors."""
        depth_append(self.K, k_layer, self.L, slot, t0, stream)
        depth_append(self.V, v_layer, self.L, slot, t0, stream)
        return self

    def tensors(self):
        """(Kd, Vd): the packed depth rows to pass to the operator with this L."""
        return self.K, self.V


class _ModaAttention(torch.autograd.Function):
    """The operator as one differentiable call: moda_fwd forward, moda_bwd backward."""

    @staticmethod
    def forward(ctx, Q, K, V, Kd, Vd, L, scale, causal, window):
        O, lse = fwd(Q, K, V, Kd, Vd, L, scale=scale, causal=causal, window=window)
        ctx.save_for_backward(Q, K, V, Kd, Vd, O, lse)
        ctx.cfg = (L, scale, causal, window)
        return O

    @staticmethod
    def backward(ctx, dO):
        Q, K, V, Kd, Vd, O, lse = ctx.saved_tensors
        L, scale, causal, window = ctx.cfg
        dQ, dK, dV, dKd, dVd = bwd(Q, K, V, Kd, Vd, O, lse, dO.contiguous(), L, scale=scale,
                                   causal=causal, window=window)
        return dQ, dK, dV, dKd, dVd, None, None, None, None


def moda_attention(Q, K, V, Kd=None, Vd=None, L=0, scale=None, causal=True, window=0):
    """O [B,Hq,T,d] of MoDA over Q [B,Hq,T,d], K, V [B,Hk,T,d] and the packed depth rows
    Kd, Vd [B,Hk,T*L,d] (None when L = 0), differentiable with respect to all five: the
    backward is moda_bwd.  The interface of the pages' kernel call, with the depth rows
    already packed (pack_depth) and the scale defaulting to 1/sqrt(d)."""
    return _ModaAttention.apply(Q, K, V, Kd, Vd, L, scale, causal, window)
