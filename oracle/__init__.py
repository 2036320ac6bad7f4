"""CPU oracle for the Mixture-of-Depths Attention (MoDA) operator.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package; the product path
(``transformer_attention_moda_amd``) never does, and this package never imports
it.  The two share no code; they meet only through seeded inputs.

``moda_oracle.c`` holds the arithmetic: the plain definition of the operator
(one softmax over the concatenation of the causal sequence keys and the
token's own depth keys, fp64, two passes per row) and its derivative.  See the
header of that file for the passages of "Mixture-of-Depths Attention"
(arXiv 2603.15619, paper summary) and of the "moda-attention 0.1.0" PyPI page
it follows.  ``brute.py`` is a second, independent transcription that builds
the full folded mask matrix literally; the tests pin the C oracle against it
and against closed forms, library routines and invariants.

Inputs are numpy arrays: float64, float32, or uint16 holding bfloat16 bit
patterns (upcast exactly).  All five inputs (and dO) must share one storage
type.  Outputs are float64.

Every forward/backward function takes two keyword options for the variants:
``causal`` (False drops the sequence causal mask; the depth mask stays) and
``window`` (0, or W in 1..L: a token sees only the last W of its L depth slots).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moda_oracle.c")
LIB_PATH = os.path.join(_HERE, "libmoda_oracle.so")

_lib = None


def build(src: str = _SRC, out: str = LIB_PATH) -> str:
    """Compile the C oracle into ``oracle/libmoda_oracle.so`` (gcc, OpenMP)."""
    tmp = out + ".tmp"
    subprocess.check_call(
        ["gcc", "-O3", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
         "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


class _Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Hk", ctypes.c_int64),
                ("T", ctypes.c_int64), ("d", ctypes.c_int64), ("L", ctypes.c_int64),
                ("scale", ctypes.c_double), ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("window", ctypes.c_int64)]


def _bind(lib):
    P = ctypes.c_void_p
    lib.oracle_fwd_rows.argtypes = [ctypes.POINTER(_Shape), P, P, P, P, P, ctypes.c_int64,
                                    P, P, P]
    lib.oracle_fwd_rows.restype = ctypes.c_int
    lib.oracle_bwd_tokens.argtypes = [ctypes.POINTER(_Shape), ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int64, P] + [P] * 13
    lib.oracle_bwd_tokens.restype = ctypes.c_int
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


class use_library:
    """Context manager that routes the wrappers to another build of the oracle
    source (the tests use it to plant mistakes in a copy and check that the pins
    catch them)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _load()
        _lib = _bind(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def num_threads() -> int:
    return int(_load().oracle_num_threads())


_CODES = {np.dtype(np.uint16): 0, np.dtype(np.float32): 1, np.dtype(np.float64): 2}


def _prep(Q, K, V, Kd, Vd, L, scale, dO=None, causal=True, window=0):
    arrs = [np.ascontiguousarray(a) for a in (Q, K, V)]
    B, Hq, T, d = arrs[0].shape
    Hk = arrs[1].shape[1]
    code = _CODES.get(arrs[0].dtype)
    if code is None:
        raise TypeError(f"unsupported storage type {arrs[0].dtype}")
    if L > 0:
        dep = [np.ascontiguousarray(Kd), np.ascontiguousarray(Vd)]
        for a in dep:
            if a.shape != (B, Hk, T * L, d):
                raise ValueError(f"depth shape {a.shape} != {(B, Hk, T * L, d)}")
    else:
        dep = [np.zeros(1, arrs[0].dtype), np.zeros(1, arrs[0].dtype)]
    arrs += dep
    if dO is not None:
        arrs.append(np.ascontiguousarray(dO))
        if arrs[-1].shape != arrs[0].shape:
            raise ValueError("dO shape must equal Q shape")
    for a in arrs:
        if a.dtype != arrs[0].dtype:
            raise TypeError("all inputs must share one storage type")
    if arrs[1].shape != (B, Hk, T, d) or arrs[2].shape != (B, Hk, T, d) or Hq % Hk:
        raise ValueError("bad K/V shape")
    if not 0 <= window <= L:
        raise ValueError(f"window {window} outside 0..L")
    shape = _Shape(B, Hq, Hk, T, d, L, float(scale), code, 0 if causal else 1, int(window))
    return shape, arrs


def _p(a):
    return ctypes.c_void_p(a.ctypes.data)


def fwd_rows(Q, K, V, Kd, Vd, L, scale, rows, causal=True, window=0):
    """Forward for selected query rows.  rows: int array [n, 3] of (b, h, t).
    Returns (O [n, d], lse [n]) in float64."""
    shape, (q, k, v, kd, vd) = _prep(Q, K, V, Kd, Vd, L, scale, causal=causal, window=window)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    n, d = rows.shape[0], shape.d
    O = np.empty((n, d), np.float64)
    lse = np.empty(n, np.float64)
    rc = _load().oracle_fwd_rows(ctypes.byref(shape), _p(q), _p(k), _p(v), _p(kd), _p(vd), n,
                                 _p(rows), _p(O), _p(lse))
    if rc != 0:
        raise ValueError("oracle_fwd_rows rejected its arguments")
    return O, lse


def fwd(Q, K, V, Kd, Vd, L, scale, causal=True, window=0):
    """Full forward: O [B,Hq,T,d] and lse [B,Hq,T] in float64."""
    B, Hq, T, d = Q.shape
    b, h, t = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(T), indexing="ij")
    rows = np.stack([b.ravel(), h.ravel(), t.ravel()], axis=1)
    O, lse = fwd_rows(Q, K, V, Kd, Vd, L, scale, rows, causal, window)
    return O.reshape(B, Hq, T, d), lse.reshape(B, Hq, T)


def bwd_tokens(Q, K, V, Kd, Vd, dO, L, scale, b, kv, tokens, causal=True, window=0):
    """Backward restricted to the rows of KV group (b, kv) at the given distinct tokens.

    Returns a dict of float64 arrays: dQ [G, n, d] (query heads kv*G .. kv*G+G-1),
    dK, dV [T, d] (contributions of the selected rows), dKd, dVd [n*L, d] (depth rows
    of the selected tokens, in the given order), O [G, n, d], lse [G, n].  When dO is
    zero at every other token of the group, dK and dV are the group's complete
    gradients (rows with zero upstream gradient contribute nothing)."""
    shape, (q, k, v, kd, vd, do) = _prep(Q, K, V, Kd, Vd, L, scale, dO, causal, window)
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64).ravel())
    if len(np.unique(tok)) != len(tok):
        raise ValueError("tokens must be distinct")
    T, d = shape.T, shape.d
    G, n = shape.Hq // shape.Hk, len(tok)
    out = dict(dQ=np.empty((G, n, d)), dK=np.empty((T, d)), dV=np.empty((T, d)),
               dKd=np.empty((max(n * L, 1), d)), dVd=np.empty((max(n * L, 1), d)),
               O=np.empty((G, n, d)), lse=np.empty((G, n)))
    rc = _load().oracle_bwd_tokens(
        ctypes.byref(shape), int(b), int(kv), n, _p(tok), _p(q), _p(k), _p(v), _p(kd),
        _p(vd), _p(do), *[_p(out[x]) for x in ("dQ", "dK", "dV", "dKd", "dVd", "O", "lse")])
    if rc != 0:
        raise ValueError("oracle_bwd_tokens rejected its arguments")
    out["dKd"] = out["dKd"][: n * L]
    out["dVd"] = out["dVd"][: n * L]
    return out


def bwd_group(Q, K, V, Kd, Vd, dO, L, scale, b, kv, t_lo=0, t_hi=None, causal=True, window=0):
    """Backward restricted to the rows of KV group (b, kv) at tokens [t_lo, t_hi).

    Returns a dict of float64 arrays: dQ [G, n, d], dK, dV [t_hi, d] (contributions of
    the selected rows; with causal masking no key past t_hi - 1 receives any), dKd, dVd
    [n*L, d] (depth rows of the selected tokens), O [G, n, d], lse [G, n]."""
    T = Q.shape[2]
    t_hi = T if t_hi is None else int(t_hi)
    if not 0 <= int(t_lo) < t_hi <= T:
        raise ValueError("bad token range")
    out = bwd_tokens(Q, K, V, Kd, Vd, dO, L, scale, b, kv, np.arange(int(t_lo), t_hi), causal,
                     window)
    if causal:
        out["dK"] = out["dK"][:t_hi]
        out["dV"] = out["dV"][:t_hi]
    return out


def bwd(Q, K, V, Kd, Vd, dO, L, scale, causal=True, window=0):
    """Full backward: dict of dQ, dK, dV, dKd, dVd (input layouts), O, lse; float64."""
    B, Hq, T, d = Q.shape
    Hk = K.shape[1]
    G = Hq // Hk
    res = dict(dQ=np.empty((B, Hq, T, d)), dK=np.empty((B, Hk, T, d)),
               dV=np.empty((B, Hk, T, d)), dKd=np.empty((B, Hk, T * L, d)),
               dVd=np.empty((B, Hk, T * L, d)), O=np.empty((B, Hq, T, d)),
               lse=np.empty((B, Hq, T)))
    for b in range(B):
        for kv in range(Hk):
            r = bwd_group(Q, K, V, Kd, Vd, dO, L, scale, b, kv, causal=causal, window=window)
            res["dQ"][b, kv * G:(kv + 1) * G] = r["dQ"]
            res["O"][b, kv * G:(kv + 1) * G] = r["O"]
            res["lse"][b, kv * G:(kv + 1) * G] = r["lse"]
            res["dK"][b, kv] = r["dK"]
            res["dV"][b, kv] = r["dV"]
            res["dKd"][b, kv] = r["dKd"]
            res["dVd"][b, kv] = r["dVd"]
    return res


def pack_depth(layers):
    """Layer-major depth KV [L, B, Hk, T, d] -> the token-major layout [B, Hk, T*L, d]
    in which row t*L + l holds layer l's entry for token t: the "Flash-compatible depth-KV
    layout" of the paper summary ("Hardware-Efficient Implementation").  A pure index
    permutation, so the result is bit-exact in any storage type."""
    L, B, Hk, T, d = layers.shape
    return np.ascontiguousarray(np.transpose(layers, (1, 2, 3, 0, 4))).reshape(B, Hk, T * L, d)


def decode(q, K, V, Kd, Vd, L, scale, pos, window=0):
    """One new query token at position `pos` attending to a cache: the sequence keys
    0..pos of K/V [B,Hk,T,d] (T = cache capacity) and its own depth rows pos*L + l of
    Kd/Vd [B,Hk,T*L,d].  q: [B,Hq,d].  Returns (O [B,Hq,d], lse [B,Hq]) in float64.
    This is exactly the forward's row at token pos (the decoding step of the paper
    summary's complexity analysis): the row is computed by the same forward routine
    with q placed at token pos."""
    B, Hq, d = q.shape
    T = K.shape[2]
    if not 0 <= pos < T:
        raise ValueError("pos outside the cache")
    Q = np.zeros((B, Hq, T, d), q.dtype)
    Q[:, :, pos] = q
    rows = np.array([[b, h, pos] for b in range(B) for h in range(Hq)], np.int64)
    O, lse = fwd_rows(Q, K, V, Kd, Vd, L, scale, rows, True, window)
    return O.reshape(B, Hq, d), lse.reshape(B, Hq)


def depth_append(packed, layer, L, slot, t0=0):
    """Write one layer's depth entries into slot `slot` of a token-major depth cache
    (the DepthKVCache role in the PyPI page's architecture list): packed [B,Hk,T*L,d],
    layer [B,Hk,n,d] holding tokens t0 .. t0+n-1.  Row (t0+i)*L + slot of each (b, kv)
    block becomes layer[b, kv, i]; every other row keeps its value.  Returns the updated
    copy (bit-exact in any storage type)."""
    B, Hk, TL, d = packed.shape
    n = layer.shape[2]
    if TL % L or layer.shape != (B, Hk, n, d) or not 0 <= slot < L or t0 < 0 or t0 + n > TL // L:
        raise ValueError("layer, slot or token range does not fit the cache")
    out = packed.copy()
    out[:, :, (t0 + np.arange(n)) * L + slot, :] = layer
    return out
