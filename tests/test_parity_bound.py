"""The edge-shape tolerance helper (CPU only): oracle.brute.abs_terms against explicit
loops over the definition's terms, and the first-order claim the bound rests on -- a
sum whose weights are rounded to bfloat16 before the products stays within 2^-8 times
the sum of the absolute terms of the exact sum."""
import math

import numpy as np
import torch

import oracle
from oracle import brute


def draw(rng, B, Hq, Hk, T, d, L):
    return [rng.standard_normal(s) for s in
            ((B, Hq, T, d), (B, Hk, T, d), (B, Hk, T, d), (B, Hk, T * L, d), (B, Hk, T * L, d),
             (B, Hq, T, d))]


def test_abs_terms_by_explicit_loops():
    rng = np.random.default_rng(41)
    B, G, Hk, T, d, L, sc = 1, 2, 1, 4, 3, 2, 0.6
    Q, K, V, Kd, Vd, dO = draw(rng, B, G * Hk, Hk, T, d, L)
    A = brute.abs_terms(Q, K, V, Kd, Vd, dO, L, sc)
    O, lse = oracle.fwd(Q, K, V, Kd, Vd, L, sc)
    want = {k: np.zeros_like(v) for k, v in A.items()}
    for h in range(G):
        for t in range(T):
            q, do = Q[0, h, t], dO[0, h, t]
            D = do @ O[0, h, t]
            keys = [(K, V, want["dK"], want["dV"], j) for j in range(t + 1)]
            keys += [(Kd, Vd, want["dKd"], want["dVd"], t * L + l) for l in range(L)]
            for kk, vv, gk, gv, j in keys:
                p = math.exp(sc * (q @ kk[0, 0, j]) - lse[0, h, t])
                ds = p * (do @ vv[0, 0, j] - D)
                want["O"][0, h, t] += p * np.abs(vv[0, 0, j])
                want["dQ"][0, h, t] += sc * abs(ds) * np.abs(kk[0, 0, j])
                gk[0, 0, j] += sc * abs(ds) * np.abs(q)
                gv[0, 0, j] += p * np.abs(do)
    for k in A:
        np.testing.assert_allclose(A[k], want[k], rtol=1e-12, atol=1e-14, err_msg=k)


def test_rounded_weights_stay_within_the_first_order_bound():
    rng = np.random.default_rng(42)
    u = 2.0 ** -8
    for n in (4, 64, 2048):
        a = rng.standard_normal((50, n)) * rng.exponential(1.0, (50, n))
        b = rng.standard_normal(n)
        exact = a @ b
        ar = torch.from_numpy(a).to(torch.bfloat16).double().numpy()
        err = np.abs(ar @ b - exact)
        assert np.all(err <= u * (np.abs(a) @ np.abs(b)) * (1 + 1e-12)), n
