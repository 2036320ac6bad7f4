"""Literal, dense transcription of the MoDA operator (test infrastructure only).

A second oracle, independent of ``moda_oracle.c`` in structure: it builds the
folded query matrix and the complete mask matrix exactly as written in
"Mixture-of-Depths Attention" (arXiv 2603.15619, paper summary), section 3.4
"Mixture-of-Depths Attention (MoDA): The Unified Operator":

* query rows of one KV group are folded, i_q = t*G + g (G adjacent rows share a
  KV head and a base-time index, "Group-aware depth-KV calculation");
* grouped causal mask: 0 where floor(i_q / G) >= i_k, -inf elsewhere (first
  masking bullet);
* depth matching mask: 0 where floor(i_q / G) == floor(j_d / L), -inf
  elsewhere (second masking bullet), over the flattened depth axis of length
  T*L ("Flash-compatible depth-KV layout");
* one softmax of (Q_fold [K || K_depth]^T) * scale + M, times [V || V_depth]
  (the MoDA equation).

Two variants change only the mask matrix: ``causal=False`` fills the sequence
block with zeros (every key visible; the MoDA README lists a non-causal kernel
as future work), and ``window=W`` keeps a depth column visible only if its slot
j_d mod L is one of the last W (the bounded, sliding-window depth slots of the
paper summary's section 6, mitigation status).

The backward is the textbook matrix form of a masked softmax-attention
gradient applied to the same concatenated matrices.  Dense: for tiny inputs
only (memory grows as (T*G) x (T + T*L)).
"""
from __future__ import annotations

import numpy as np


def _group(Q, K, V, Kd, Vd, L, b, kv, causal=True, window=0):
    B, Hq, T, d = Q.shape
    Hk = K.shape[1]
    G = Hq // Hk
    Qf = np.transpose(Q[b, kv * G:(kv + 1) * G], (1, 0, 2)).reshape(T * G, d)
    if L > 0:
        keys = np.concatenate([K[b, kv], Kd[b, kv]], axis=0)
        vals = np.concatenate([V[b, kv], Vd[b, kv]], axis=0)
    else:
        keys, vals = K[b, kv], V[b, kv]
    iq = np.arange(T * G)[:, None]
    ik = np.arange(T)[None, :]
    jd = np.arange(T * L)[None, :]
    m_seq = np.where(iq // G >= ik, 0.0, -np.inf) if causal else np.zeros((T * G, T))
    W = window if window > 0 else L
    if L > 0:
        m_dep = np.where((iq // G == jd // L) & (jd % L >= L - W), 0.0, -np.inf)
    else:
        m_dep = np.zeros((T * G, 0))
    M = np.concatenate([m_seq, m_dep], axis=1)
    return Qf, keys, vals, M, G, T


def _unfold(x, G, T):
    """[T*G, ...] folded rows -> [G, T, ...]."""
    return np.swapaxes(x.reshape((T, G) + x.shape[1:]), 0, 1)


def forward(Q, K, V, Kd, Vd, L, scale, causal=True, window=0):
    """O [B,Hq,T,d], lse [B,Hq,T] (float64) from float64 inputs."""
    B, Hq, T, d = Q.shape
    Hk = K.shape[1]
    G = Hq // Hk
    O = np.zeros((B, Hq, T, d))
    lse = np.zeros((B, Hq, T))
    for b in range(B):
        for kv in range(Hk):
            Qf, keys, vals, M, G, T = _group(Q, K, V, Kd, Vd, L, b, kv, causal, window)
            S = (Qf @ keys.T) * scale + M
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            Z = E.sum(axis=1, keepdims=True)
            P = E / Z
            O[b, kv * G:(kv + 1) * G] = _unfold(P @ vals, G, T)
            lse[b, kv * G:(kv + 1) * G] = _unfold((m + np.log(Z))[:, 0], G, T)
    return O, lse


def backward(Q, K, V, Kd, Vd, dO, L, scale, causal=True, window=0):
    """dQ, dK, dV, dKd, dVd (float64) from float64 inputs."""
    B, Hq, T, d = Q.shape
    Hk = K.shape[1]
    G = Hq // Hk
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    dKd = np.zeros((B, Hk, T * L, d))
    dVd = np.zeros((B, Hk, T * L, d))
    for b in range(B):
        for kv in range(Hk):
            Qf, keys, vals, M, G, T = _group(Q, K, V, Kd, Vd, L, b, kv, causal, window)
            dOf = np.transpose(dO[b, kv * G:(kv + 1) * G], (1, 0, 2)).reshape(T * G, d)
            S = (Qf @ keys.T) * scale + M
            E = np.exp(S - S.max(axis=1, keepdims=True))
            P = E / E.sum(axis=1, keepdims=True)
            Of = P @ vals
            dP = dOf @ vals.T
            dS = P * (dP - (dOf * Of).sum(axis=1, keepdims=True))
            dQ[b, kv * G:(kv + 1) * G] = _unfold(scale * dS @ keys, G, T)
            dkeys = scale * dS.T @ Qf
            dvals = P.T @ dOf
            dK[b, kv], dV[b, kv] = dkeys[:T], dvals[:T]
            if L > 0:
                dKd[b, kv], dVd[b, kv] = dkeys[T:], dvals[T:]
    return dQ, dK, dV, dKd, dVd


def abs_terms(Q, K, V, Kd, Vd, dO, L, scale, causal=True, window=0):
    """Per output element, the sum of the absolute values of the terms of the product that
    yields it (exact fp64 weights): O = P V -> P |V|; dV, dVd = P^T dO -> P^T |dO|;
    dQ = scale dS [K||Kd] -> scale |dS| [|K|||Kd|]; dK, dKd = scale dS^T Q -> scale
    |dS|^T |Q|.  A product whose left operand is rounded to a format of unit roundoff u
    before an exactly accumulated sum is off by at most u times this (first order), which
    sizes the tolerance of outputs that are sums of many such terms.  Dict keyed like the
    outputs (dO may be None: forward only)."""
    B, Hq, T, d = Q.shape
    Hk = K.shape[1]
    G = Hq // Hk
    out = {"O": np.zeros((B, Hq, T, d))}
    if dO is not None:
        out.update(dQ=np.zeros_like(Q), dK=np.zeros_like(K), dV=np.zeros_like(V),
                   dKd=np.zeros((B, Hk, T * L, d)), dVd=np.zeros((B, Hk, T * L, d)))
    for b in range(B):
        for kv in range(Hk):
            Qf, keys, vals, M, G, T = _group(Q, K, V, Kd, Vd, L, b, kv, causal, window)
            S = (Qf @ keys.T) * scale + M
            E = np.exp(S - S.max(axis=1, keepdims=True))
            P = E / E.sum(axis=1, keepdims=True)
            out["O"][b, kv * G:(kv + 1) * G] = _unfold(P @ np.abs(vals), G, T)
            if dO is None:
                continue
            dOf = np.transpose(dO[b, kv * G:(kv + 1) * G], (1, 0, 2)).reshape(T * G, d)
            Of = P @ vals
            dS = np.abs(P * (dOf @ vals.T - (dOf * Of).sum(axis=1, keepdims=True)))
            out["dQ"][b, kv * G:(kv + 1) * G] = _unfold(scale * dS @ np.abs(keys), G, T)
            dk = scale * dS.T @ np.abs(Qf)
            dv = P.T @ np.abs(dOf)
            out["dK"][b, kv], out["dV"][b, kv] = dk[:T], dv[:T]
            if L > 0:
                out["dKd"][b, kv], out["dVd"][b, kv] = dk[T:], dv[T:]
    return out
