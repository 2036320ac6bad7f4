"""Pins of the CPU oracle against facts other than itself (CPU only).

Each test names what fixes the expected value: a literal dense transcription
of the pages' equation and masks (oracle/brute.py), a library routine
(torch scaled_dot_product_attention, scipy softmax), a closed form, an
invariant of the definition, or central finite differences of the oracle's
own forward.  The passages are those of "Mixture-of-Depths Attention"
(arXiv 2603.15619, paper summary), section 3.4 unless stated otherwise.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import brute


def draw(rng, B, Hq, Hk, T, d, L, kd_scale=1.0):
    Q = rng.standard_normal((B, Hq, T, d))
    K = rng.standard_normal((B, Hk, T, d))
    V = rng.standard_normal((B, Hk, T, d))
    Kd = rng.standard_normal((B, Hk, T * L, d)) * kd_scale
    Vd = rng.standard_normal((B, Hk, T * L, d))
    return Q, K, V, Kd, Vd


def to_bf16_bits(x):
    """float64 -> bfloat16 bit patterns (round to nearest even) and their exact values."""
    t = torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16), t.to(torch.float64).numpy()


# --- the MoDA equation and both masks: C oracle == literal dense transcription ---

def test_forward_matches_dense_transcription_grid():
    rng = np.random.default_rng(1)
    for T, L, G, d in itertools.product((1, 2, 3, 5, 8, 13, 24), (0, 1, 2, 3), (1, 2, 4),
                                        (1, 4, 8)):
        Hk = 2 if T % 2 else 1
        B = 2 if d == 4 else 1
        args = draw(rng, B, G * Hk, Hk, T, d, L)
        scale = 1.0 / math.sqrt(d)
        O, lse = oracle.fwd(*args, L, scale)
        Ob, lseb = brute.forward(*args, L, scale)
        np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12, err_msg=f"T{T} L{L} G{G} d{d}")
        np.testing.assert_allclose(lse, lseb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("storage", ["bf16", "f32"])
def test_forward_storage_upcast_is_exact(storage):
    rng = np.random.default_rng(2)
    args = draw(rng, 1, 4, 2, 9, 8, 3)
    if storage == "bf16":
        pairs = [to_bf16_bits(a) for a in args]
        stored, exact = [p[0] for p in pairs], [p[1] for p in pairs]
    else:
        stored = [np.asarray(a, np.float32) for a in args]
        exact = [s.astype(np.float64) for s in stored]
    scale = float(np.float32(1 / math.sqrt(8)))
    O, lse = oracle.fwd(*stored, 3, scale)
    Ob, lseb = brute.forward(*exact, 3, scale)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lseb, rtol=0, atol=1e-12)


def test_forward_rows_subset_equals_full():
    rng = np.random.default_rng(3)
    args = draw(rng, 2, 4, 2, 17, 8, 2)
    O, lse = oracle.fwd(*args, 2, 0.3)
    rows = np.array([[1, 3, 16], [0, 0, 0], [1, 2, 7], [0, 1, 9]])
    Os, lses = oracle.fwd_rows(*args, 2, 0.3, rows)
    for i, (b, h, t) in enumerate(rows):
        np.testing.assert_array_equal(Os[i], O[b, h, t])
        assert lses[i] == lse[b, h, t]


# --- L = 0: MoDA reduces to causal self-attention (the depth-KV paragraph) ---

@pytest.mark.parametrize("G", [1, 2, 4])
def test_no_depth_equals_library_causal_attention(G):
    rng = np.random.default_rng(4 + G)
    Hk, T, d = 2, 33, 16
    Q, K, V, _, _ = draw(rng, 2, G * Hk, Hk, T, d, 0)
    scale = 1 / math.sqrt(d)
    O, lse = oracle.fwd(Q, K, V, None, None, 0, scale)
    q = torch.from_numpy(Q)
    # GQA expansion as the PyPI page's "Key Design Choices" states: repeat_interleave.
    k = torch.from_numpy(K).repeat_interleave(G, dim=1)
    v = torch.from_numpy(V).repeat_interleave(G, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)
    np.testing.assert_allclose(O, ref.numpy(), rtol=0, atol=1e-12)
    s = torch.einsum("bhtd,bhjd->bhtj", q, k) * scale
    s = s.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), rtol=0, atol=1e-12)


# --- closed forms ---

def test_zero_query_gives_uniform_weights():
    rng = np.random.default_rng(5)
    B, G, Hk, T, d, L = 1, 2, 2, 11, 4, 3
    _, K, V, Kd, Vd = draw(rng, B, G * Hk, Hk, T, d, L)
    Q = np.zeros((B, G * Hk, T, d))
    O, lse = oracle.fwd(Q, K, V, Kd, Vd, L, 0.5)
    for h in range(G * Hk):
        kv = h // G
        for t in range(T):
            expect = (V[0, kv, :t + 1].sum(0) + Vd[0, kv, t * L:(t + 1) * L].sum(0)) / (t + 1 + L)
            np.testing.assert_allclose(O[0, h, t], expect, rtol=0, atol=1e-13)
            assert abs(lse[0, h, t] - math.log(t + 1 + L)) < 1e-13


def test_hand_worked_two_token_example():
    # d = 1, G = 1, L = 1, scale = 1.  Token 0 sees K0 (score 1) and its depth key (score 0);
    # token 1 sees K0 (score 2), K1 (score 0) and its depth key (score 2).
    Q = np.array([1.0, 2.0]).reshape(1, 1, 2, 1)
    K = np.array([1.0, 0.0]).reshape(1, 1, 2, 1)
    V = np.array([1.0, 2.0]).reshape(1, 1, 2, 1)
    Kd = np.array([0.0, 1.0]).reshape(1, 1, 2, 1)
    Vd = np.array([3.0, 5.0]).reshape(1, 1, 2, 1)
    O, lse = oracle.fwd(Q, K, V, Kd, Vd, 1, 1.0)
    e = math.e
    assert abs(O[0, 0, 0, 0] - (e * 1 + 1 * 3) / (e + 1)) < 1e-14
    assert abs(lse[0, 0, 0] - math.log(e + 1)) < 1e-14
    assert abs(O[0, 0, 1, 0] - (e**2 * 1 + 1 * 2 + e**2 * 5) / (2 * e**2 + 1)) < 1e-14
    assert abs(lse[0, 0, 1] - math.log(2 * e**2 + 1)) < 1e-14


def test_attention_mass_sums_to_one():
    # With every value row equal to 1 the output is the total attention mass.
    rng = np.random.default_rng(6)
    Q, K, _, Kd, _ = draw(rng, 2, 4, 2, 19, 8, 5)
    ones, ones_d = np.ones((2, 2, 19, 8)), np.ones((2, 2, 19 * 5, 8))
    O, _ = oracle.fwd(Q * 3, K, ones, Kd, ones_d, 5, 0.4)
    np.testing.assert_allclose(O, 1.0, rtol=0, atol=1e-13)


# --- depth matching mask: depends only on floor(j_d / L) ---

def test_depth_slot_permutation_invariance():
    rng = np.random.default_rng(7)
    B, G, Hk, T, d, L = 1, 2, 2, 10, 8, 6
    Q, K, V, Kd, Vd = draw(rng, B, G * Hk, Hk, T, d, L)
    dO = rng.standard_normal(Q.shape)
    perm = np.concatenate([t * L + rng.permutation(L) for t in range(T)])
    O1, l1 = oracle.fwd(Q, K, V, Kd, Vd, L, 0.35)
    O2, l2 = oracle.fwd(Q, K, V, Kd[:, :, perm], Vd[:, :, perm], L, 0.35)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)
    g1 = oracle.bwd(Q, K, V, Kd, Vd, dO, L, 0.35)
    g2 = oracle.bwd(Q, K, V, Kd[:, :, perm], Vd[:, :, perm], dO, L, 0.35)
    np.testing.assert_allclose(g1["dKd"][:, :, perm], g2["dKd"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(g1["dVd"][:, :, perm], g2["dVd"], rtol=0, atol=1e-12)
    for k in ("dQ", "dK", "dV"):
        np.testing.assert_allclose(g1[k], g2[k], rtol=0, atol=1e-12)


def test_sequence_pushed_to_minus_infinity_gives_depth_attention():
    # Depth Attention (section 3.4, "Depth Attention" paragraph) attends per token over
    # the depth keys only.  Q_t = a e1 + q', K_j = -a e1 + k', depth keys orthogonal to e1:
    # every sequence score is below -a^2 * scale + O(1), depth scores are untouched.
    rng = np.random.default_rng(8)
    B, G, Hk, T, d, L, a = 1, 2, 1, 12, 8, 5, 30.0
    Q, K, V, Kd, Vd = draw(rng, B, G * Hk, Hk, T, d, L)
    Q[..., 0], K[..., 0], Kd[..., 0] = a, -a, 0.0
    scale = 1 / math.sqrt(d)
    O, lse = oracle.fwd(Q, K, V, Kd, Vd, L, scale)
    for h in range(G * Hk):
        for t in range(T):
            u = scale * Kd[0, 0, t * L:(t + 1) * L] @ Q[0, h, t]
            w = scipy.special.softmax(u)
            np.testing.assert_allclose(O[0, h, t], w @ Vd[0, 0, t * L:(t + 1) * L], rtol=0,
                                       atol=1e-12)
            assert abs(lse[0, h, t] - scipy.special.logsumexp(u)) < 1e-12


# --- the fused online-softmax reading ("Fused online-softmax (Algorithm 1)") ---

def online_moda_row_group(Q, K, V, Kd, Vd, L, scale, b, kv, block_q, block_k):
    """Blockwise base-2 online softmax over folded rows: unmasked sequence blocks,
    boundary blocks with the grouped causal mask, then depth blocks with the depth
    matching mask, all updating one (m, acc, o) state per row."""
    B, Hq, T, d = Q.shape
    G = Hq // K.shape[1]
    log2e = 1.0 / math.log(2.0)
    Qf = np.transpose(Q[b, kv * G:(kv + 1) * G], (1, 0, 2)).reshape(T * G, d)
    out = np.zeros((T * G, d))
    lse = np.zeros(T * G)
    for r0 in range(0, T * G, block_q):
        rows = np.arange(r0, min(r0 + block_q, T * G))
        tb = rows // G
        t_start, t_end = tb.min(), tb.max() + 1
        m = np.full(len(rows), -np.inf)
        acc = np.zeros(len(rows))
        o = np.zeros((len(rows), d))

        def update(S):
            nonlocal m, acc, o
            m_new = np.maximum(m, S.max(axis=1))
            alpha = np.exp2(m - m_new)
            Pb = np.exp2(S - m_new[:, None])
            return m_new, alpha, Pb

        for k0 in range(0, t_end, block_k):
            ks = np.arange(k0, min(k0 + block_k, t_end))
            S = (Qf[rows] @ K[b, kv, ks].T) * scale * log2e
            if ks[-1] >= t_start:
                S = np.where(tb[:, None] >= ks[None, :], S, -np.inf)
            m_new, alpha, Pb = update(S)
            acc = acc * alpha + Pb.sum(1)
            o = o * alpha[:, None] + Pb @ V[b, kv, ks]
            m = m_new
        for j0 in range(t_start * L, t_end * L, block_k):
            js = np.arange(j0, min(j0 + block_k, t_end * L))
            S = (Qf[rows] @ Kd[b, kv, js].T) * scale * log2e
            S = np.where(tb[:, None] == js[None, :] // L, S, -np.inf)
            m_new, alpha, Pb = update(S)
            acc = acc * alpha + Pb.sum(1)
            o = o * alpha[:, None] + Pb @ Vd[b, kv, js]
            m = m_new
        out[rows] = o / acc[:, None]
        lse[rows] = (m + np.log2(acc)) / log2e
    return out, lse


@pytest.mark.parametrize("block_q,block_k", [(4, 3), (8, 16), (6, 5)])
def test_online_blockwise_reading_equals_two_pass(block_q, block_k):
    rng = np.random.default_rng(9)
    B, G, Hk, T, d, L = 1, 2, 2, 23, 8, 3
    args = draw(rng, B, G * Hk, Hk, T, d, L)
    O, lse = oracle.fwd(*args, L, 0.3)
    for kv in range(Hk):
        of, lf = online_moda_row_group(*args, L, 0.3, 0, kv, block_q, block_k)
        for g in range(G):
            np.testing.assert_allclose(O[0, kv * G + g], of[g::G], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[0, kv * G + g], lf[g::G], rtol=0, atol=1e-12)


# --- backward ---

def loss(args, dO, L, scale):
    O, _ = oracle.fwd(*args, L, scale)
    return float((O * dO).sum())


def test_backward_matches_central_finite_differences():
    rng = np.random.default_rng(10)
    B, G, Hk, T, d, L, scale = 1, 2, 2, 6, 3, 2, 0.7
    args = list(draw(rng, B, G * Hk, Hk, T, d, L))
    dO = rng.standard_normal(args[0].shape)
    g = oracle.bwd(*args, dO, L, scale)
    names = ["dQ", "dK", "dV", "dKd", "dVd"]
    h = 1e-6
    for ti, name in enumerate(names):
        x = args[ti]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = loss(args, dO, L, scale)
            x[idx] = old - h
            lm = loss(args, dO, L, scale)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.linalg.norm(g[name] - num) / np.linalg.norm(num)
        assert err < 1e-6, (name, err)


def test_backward_matches_dense_transcription_grid():
    rng = np.random.default_rng(11)
    for T, L, G in itertools.product((1, 4, 9), (0, 1, 3), (1, 2, 4)):
        args = draw(rng, 1, 2 * G, 2, T, 4, L)
        dO = rng.standard_normal(args[0].shape)
        g = oracle.bwd(*args, dO, L, 0.45)
        ref = brute.backward(*args, dO, L, 0.45)
        for name, r in zip(("dQ", "dK", "dV", "dKd", "dVd"), ref):
            np.testing.assert_allclose(g[name], r, rtol=0, atol=1e-11, err_msg=name)


@pytest.mark.parametrize("G", [1, 2])
def test_backward_no_depth_equals_library_autograd(G):
    rng = np.random.default_rng(12)
    Hk, T, d = 2, 21, 8
    Q, K, V, _, _ = draw(rng, 1, G * Hk, Hk, T, d, 0)
    dO = rng.standard_normal(Q.shape)
    g = oracle.bwd(Q, K, V, None, None, dO, 0, 0.3)
    q, k, v = (torch.from_numpy(x).requires_grad_() for x in (Q, K, V))
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(G, 1), v.repeat_interleave(G, 1), is_causal=True, scale=0.3)
    o.backward(torch.from_numpy(dO))
    np.testing.assert_allclose(g["dQ"], q.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dK"], k.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dV"], v.grad.numpy(), rtol=0, atol=1e-12)


def test_backward_invariants():
    rng = np.random.default_rng(13)
    B, G, Hk, T, d, L = 2, 2, 2, 14, 6, 4
    Q, K, V, Kd, Vd = draw(rng, B, G * Hk, Hk, T, d, L)
    dO = rng.standard_normal(Q.shape)
    g = oracle.bwd(Q, K, V, Kd, Vd, dO, L, 0.5)
    for b in range(B):
        for kv in range(Hk):
            grp = slice(kv * G, (kv + 1) * G)
            # shifting every key of the group by one vector shifts each row's scores by a constant
            np.testing.assert_allclose(g["dK"][b, kv].sum(0) + g["dKd"][b, kv].sum(0), 0,
                                       atol=1e-11)
            # adding one vector to every value adds it to every output row
            np.testing.assert_allclose(g["dV"][b, kv].sum(0) + g["dVd"][b, kv].sum(0),
                                       dO[b, grp].sum((0, 1)), atol=1e-11)
            # scaling queries by c and keys by 1/c leaves every score unchanged
            lhs = (Q[b, grp] * g["dQ"][b, grp]).sum()
            rhs = (K[b, kv] * g["dK"][b, kv]).sum() + (Kd[b, kv] * g["dKd"][b, kv]).sum()
            assert abs(lhs - rhs) < 1e-10


def test_depth_gradients_are_token_local():
    rng = np.random.default_rng(14)
    B, G, Hk, T, d, L = 1, 2, 1, 8, 4, 3
    Q, K, V, Kd, Vd = draw(rng, B, G * Hk, Hk, T, d, L)
    dO = rng.standard_normal(Q.shape)
    g1 = oracle.bwd(Q, K, V, Kd, Vd, dO, L, 0.5)
    dO2 = dO.copy()
    dO2[:, :, 5] += 1.0
    g2 = oracle.bwd(Q, K, V, Kd, Vd, dO2, L, 0.5)
    keep = np.ones(T * L, bool)
    keep[5 * L:6 * L] = False
    np.testing.assert_array_equal(g1["dKd"][:, :, keep], g2["dKd"][:, :, keep])
    np.testing.assert_array_equal(g1["dVd"][:, :, keep], g2["dVd"][:, :, keep])
    assert not np.allclose(g1["dVd"][:, :, ~keep], g2["dVd"][:, :, ~keep])


def test_backward_token_range_restriction():
    rng = np.random.default_rng(15)
    B, G, Hk, T, d, L = 1, 2, 2, 20, 4, 2
    args = draw(rng, B, G * Hk, Hk, T, d, L)
    dO = rng.standard_normal(args[0].shape)
    full = oracle.bwd(*args, dO, L, 0.5)
    t_lo = 13
    part = oracle.bwd_group(*args, dO, L, 0.5, b=0, kv=1, t_lo=t_lo, t_hi=T)
    np.testing.assert_allclose(part["dQ"], full["dQ"][0, 2:4, t_lo:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(part["dK"][t_lo:], full["dK"][0, 1, t_lo:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(part["dV"][t_lo:], full["dV"][0, 1, t_lo:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(part["dKd"], full["dKd"][0, 1, t_lo * L:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(part["dVd"], full["dVd"][0, 1, t_lo * L:], rtol=0, atol=1e-13)


def test_pack_depth_row_order_by_explicit_loops():
    """The packer's layout, element by element: token t's slot l is row t*L + l of its
    (batch, KV head) block, and nothing else moves (paper summary, flash-compatible
    depth-KV layout)."""
    rng = np.random.default_rng(5)
    for (L, B, Hk, T, d) in [(3, 2, 2, 5, 4), (1, 1, 1, 1, 8), (4, 1, 3, 2, 1)]:
        layers = rng.integers(0, 1 << 16, size=(L, B, Hk, T, d), dtype=np.uint16)
        got = oracle.pack_depth(layers)
        assert got.shape == (B, Hk, T * L, d) and got.dtype == layers.dtype
        want = np.empty_like(got)
        for l in range(L):
            for b in range(B):
                for h in range(Hk):
                    for t in range(T):
                        want[b, h, t * L + l, :] = layers[l, b, h, t, :]
        assert np.array_equal(got, want)


# --- variants: non-causal sequence keys, sliding-window depth slots ---

def test_variants_match_dense_transcription_grid():
    """Non-causal (the MoDA README's future-work kernel, read as: drop the sequence causal
    mask, keep the depth matching mask) and the depth window (paper summary, section 6,
    bounded depth-KV slots with a sliding-window recency policy: the last W slots), fwd
    and bwd, against the literal mask matrix of oracle/brute.py."""
    rng = np.random.default_rng(21)
    for T, L, G, causal in itertools.product((1, 3, 8, 13), (0, 1, 3, 5), (1, 2, 4),
                                             (True, False)):
        for W in sorted({0, 1, L} | ({L - 1} if L > 1 else set())):
            if W > L:
                continue
            args = draw(rng, 1, 2 * G, 2, T, 4, L)
            dO = rng.standard_normal(args[0].shape)
            tag = f"T{T} L{L} G{G} causal={causal} W={W}"
            O, lse = oracle.fwd(*args, L, 0.45, causal=causal, window=W)
            Ob, lb = brute.forward(*args, L, 0.45, causal=causal, window=W)
            np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12, err_msg=tag)
            np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12, err_msg=tag)
            g = oracle.bwd(*args, dO, L, 0.45, causal=causal, window=W)
            ref = brute.backward(*args, dO, L, 0.45, causal=causal, window=W)
            for name, r in zip(("dQ", "dK", "dV", "dKd", "dVd"), ref):
                np.testing.assert_allclose(g[name], r, rtol=0, atol=1e-11, err_msg=f"{tag} {name}")


@pytest.mark.parametrize("G", [1, 4])
def test_noncausal_no_depth_equals_library_attention(G):
    """With L = 0 the non-causal operator is plain bidirectional GQA attention: torch's
    scaled_dot_product_attention without the causal mask, forward and autograd."""
    rng = np.random.default_rng(22)
    Hk, T, d = 2, 17, 8
    Q, K, V, _, _ = draw(rng, 1, G * Hk, Hk, T, d, 0)
    dO = rng.standard_normal(Q.shape)
    O, lse = oracle.fwd(Q, K, V, None, None, 0, 0.3, causal=False)
    g = oracle.bwd(Q, K, V, None, None, dO, 0, 0.3, causal=False)
    q, k, v = (torch.from_numpy(x).requires_grad_() for x in (Q, K, V))
    kr, vr = k.repeat_interleave(G, 1), v.repeat_interleave(G, 1)
    o = torch.nn.functional.scaled_dot_product_attention(q, kr, vr, is_causal=False, scale=0.3)
    o.backward(torch.from_numpy(dO))
    ref_lse = torch.logsumexp(0.3 * q.detach() @ kr.detach().transpose(-1, -2), -1)
    np.testing.assert_allclose(O, o.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dQ"], q.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dK"], k.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dV"], v.grad.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("W", [1, 3, 5])
def test_window_equals_operator_on_truncated_depth_cache(causal, W):
    """Seeing only the last W of L slots is the plain operator on a depth cache that
    holds just those W slots per token (L' = W); the hidden slots get zero gradient.
    W = L is the plain operator itself."""
    rng = np.random.default_rng(23)
    B, G, Hk, T, d, L = 1, 2, 2, 11, 6, 5
    Q, K, V, Kd, Vd = draw(rng, B, G * Hk, Hk, T, d, L)
    dO = rng.standard_normal(Q.shape)
    keep = (np.arange(T)[:, None] * L + np.arange(L - W, L)[None, :]).ravel()
    Kt, Vt = Kd[:, :, keep], Vd[:, :, keep]
    O, lse = oracle.fwd(Q, K, V, Kd, Vd, L, 0.4, causal=causal, window=W)
    Ot, lt = oracle.fwd(Q, K, V, Kt, Vt, W, 0.4, causal=causal)
    np.testing.assert_allclose(O, Ot, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lt, rtol=0, atol=1e-13)
    g = oracle.bwd(Q, K, V, Kd, Vd, dO, L, 0.4, causal=causal, window=W)
    gt = oracle.bwd(Q, K, V, Kt, Vt, dO, W, 0.4, causal=causal)
    for k in ("dQ", "dK", "dV"):
        np.testing.assert_allclose(g[k], gt[k], rtol=0, atol=1e-12)
    for k in ("dKd", "dVd"):
        np.testing.assert_allclose(g[k][:, :, keep], gt[k], rtol=0, atol=1e-12)
        hidden = np.ones(T * L, bool)
        hidden[keep] = False
        assert np.all(g[k][:, :, hidden] == 0.0)


def test_variant_backward_matches_central_finite_differences():
    rng = np.random.default_rng(24)
    B, G, Hk, T, d, L, scale = 1, 2, 1, 5, 3, 3, 0.6
    args = list(draw(rng, B, G * Hk, Hk, T, d, L))
    dO = rng.standard_normal(args[0].shape)
    for causal, W in ((False, 0), (True, 2), (False, 1)):
        g = oracle.bwd(*args, dO, L, scale, causal=causal, window=W)
        h = 1e-6
        for ti, name in enumerate(("dQ", "dK", "dV", "dKd", "dVd")):
            x = args[ti]
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                old = x[idx]
                x[idx] = old + h
                lp = float((oracle.fwd(*args, L, scale, causal, W)[0] * dO).sum())
                x[idx] = old - h
                lm = float((oracle.fwd(*args, L, scale, causal, W)[0] * dO).sum())
                x[idx] = old
                num[idx] = (lp - lm) / (2 * h)
            err = np.linalg.norm(g[name] - num) / max(np.linalg.norm(num), 1e-300)
            assert err < 1e-6 or np.linalg.norm(g[name] - num) < 1e-9, (causal, W, name, err)


# --- the token-set backward: complete key gradients under a sparse upstream gradient ---

@pytest.mark.parametrize("causal", [True, False])
def test_sparse_upstream_gradient_token_set_backward_is_complete(causal):
    """Rows whose upstream gradient is zero contribute nothing to dK and dV (their dS and
    p*dO vanish), so with dO zero outside a token set the restricted backward over that set
    gives the complete key gradients; its dQ rows and the set's depth rows are complete in
    any case."""
    rng = np.random.default_rng(25)
    B, G, Hk, T, d, L = 1, 2, 2, 19, 5, 3
    Q, K, V, Kd, Vd = draw(rng, B, G * Hk, Hk, T, d, L)
    tokens = np.array([17, 0, 9, 4, 18])           # any order
    dO = np.zeros(Q.shape)
    dO[:, :, tokens] = rng.standard_normal((B, G * Hk, len(tokens), d))
    full = oracle.bwd(Q, K, V, Kd, Vd, dO, L, 0.5, causal=causal, window=2)
    for kv in range(Hk):
        part = oracle.bwd_tokens(Q, K, V, Kd, Vd, dO, L, 0.5, 0, kv, tokens, causal=causal,
                                 window=2)
        np.testing.assert_allclose(part["dK"], full["dK"][0, kv], rtol=0, atol=1e-13)
        np.testing.assert_allclose(part["dV"], full["dV"][0, kv], rtol=0, atol=1e-13)
        np.testing.assert_allclose(part["dQ"], full["dQ"][0, kv * G:(kv + 1) * G][:, tokens],
                                   rtol=0, atol=1e-13)
        rows = (tokens[:, None] * L + np.arange(L)[None, :]).ravel()
        np.testing.assert_allclose(part["dKd"], full["dKd"][0, kv, rows], rtol=0, atol=1e-13)
        np.testing.assert_allclose(part["dVd"], full["dVd"][0, kv, rows], rtol=0, atol=1e-13)


# --- decoding and the append-mode depth cache ---

def test_decode_is_the_forward_row_of_the_new_token():
    """Decoding one token (paper summary, complexity analysis: one new token attends over
    the cached sequence keys and its own depth keys) is the forward's row at that token:
    the dense transcription's last row of the sequence that ends with it.  Cache entries
    past the token's position must not matter."""
    rng = np.random.default_rng(26)
    B, G, Hk, Tcap, d, L = 2, 4, 2, 12, 8, 3
    _, K, V, Kd, Vd = draw(rng, B, G * Hk, Hk, Tcap, d, L)
    q = rng.standard_normal((B, G * Hk, d))
    for pos, W in ((0, 0), (5, 2), (Tcap - 1, 0)):
        O, lse = oracle.decode(q, K, V, Kd, Vd, L, 0.35, pos, window=W)
        n = pos + 1
        Qs = rng.standard_normal((B, G * Hk, n, d))
        Qs[:, :, pos] = q
        Ob, lb = brute.forward(Qs, K[:, :, :n], V[:, :, :n], Kd[:, :, :n * L], Vd[:, :, :n * L],
                               L, 0.35, window=W)
        np.testing.assert_allclose(O, Ob[:, :, pos], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lb[:, :, pos], rtol=0, atol=1e-12)


def test_depth_append_builds_the_packed_cache():
    """Appending layer l's entries into slot l for l = 0..L-1 gives exactly the packed
    token-major layout (pack_depth of the stacked layers); a ranged append writes only
    rows (t0+i)*L + slot, by explicit loops."""
    rng = np.random.default_rng(27)
    L, B, Hk, T, d = 4, 2, 3, 6, 8
    layers = rng.integers(0, 1 << 16, size=(L, B, Hk, T, d), dtype=np.uint16)
    cache = np.zeros((B, Hk, T * L, d), np.uint16)
    for l in range(L):
        cache = oracle.depth_append(cache, layers[l], L, l)
    assert np.array_equal(cache, oracle.pack_depth(layers))
    new = rng.integers(0, 1 << 16, size=(B, Hk, 2, d), dtype=np.uint16)
    got = oracle.depth_append(cache, new, L, 1, t0=3)
    want = cache.copy()
    for b in range(B):
        for h in range(Hk):
            for i in range(2):
                want[b, h, (3 + i) * L + 1, :] = new[b, h, i, :]
    assert np.array_equal(got, want)
    with pytest.raises(ValueError):
        oracle.depth_append(cache, new, L, 1, t0=5)
