"""Pins of the backward oracle against facts it does not define itself.

Finite differences of the forward oracle (plan frozen), a library routine for
the dense limit (torch fp64 autograd), invariants of softmax attention and
special cases where the Taylor route is exact.  No GPU is involved.
"""

import numpy as np
import pytest
import torch

from oracle import isa_oracle as orc
from oracle import isa_oracle_backward as bwd


def _inputs(Ns, Nc, d, seed, ctx_scale=0.5):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((Ns, d))
    K = rng.standard_normal((Ns + Nc, d))
    K[Ns:] *= ctx_scale
    V = rng.standard_normal((Ns + Nc, d))
    dO = rng.standard_normal((Ns, d))
    return Q, K, V, dO


def _plan(Q, K, V, b, rho, gamma):
    p = orc.oracle_plan_head(Q, K, V, b, rho, gamma)
    return p["kept_ctx"], p["full_q"]


def _loss(Q, K, V, dO, b, kept, full):
    return float((dO * orc.oracle_forward_head(Q, K, V, b, kept, full)).sum())


CASES = [
    # Ns, Nc, d, b, rho, gamma
    (13, 11, 4, 3, 0.5, 0.4),    # ragged tails in both segments
    (10, 0, 3, 4, 0.5, 0.5),     # no context
    (9, 7, 3, 2, 0.0, 0.5),      # every context block pruned
    (12, 9, 4, 3, 1.0, 0.0),     # Taylor only
    (12, 9, 4, 3, 0.5, 1.0),     # full only
    (8, 6, 3, 1, 0.5, 0.5),      # b = 1
    (7, 5, 3, 16, 1.0, 0.0),     # b larger than both segments
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "Ns%d_Nc%d_d%d_b%d_r%g_g%g" % c)
def test_directional_finite_differences(case):
    Ns, Nc, d, b, rho, gamma = case
    Q, K, V, dO = _inputs(Ns, Nc, d, seed=Ns * 31 + Nc)
    kept, full = _plan(Q, K, V, b, rho, gamma)
    dQ, dK, dV = bwd.oracle_backward_head(Q, K, V, dO, b, kept, full)
    rng = np.random.default_rng(7)
    eps = 1e-6
    for _ in range(4):
        EQ, EK, EV = rng.standard_normal(Q.shape), rng.standard_normal(K.shape), rng.standard_normal(V.shape)
        lp = _loss(Q + eps * EQ, K + eps * EK, V + eps * EV, dO, b, kept, full)
        lm = _loss(Q - eps * EQ, K - eps * EK, V - eps * EV, dO, b, kept, full)
        fd = (lp - lm) / (2 * eps)
        an = (dQ * EQ).sum() + (dK * EK).sum() + (dV * EV).sum()
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (fd, an)


def test_elementwise_finite_differences():
    Ns, Nc, d, b = 7, 5, 3, 2
    Q, K, V, dO = _inputs(Ns, Nc, d, seed=3)
    kept, full = _plan(Q, K, V, b, 0.5, 0.5)
    assert 0 < len(full) < (Ns + b - 1) // b and 0 < len(kept) < (Nc + b - 1) // b
    grads = bwd.oracle_backward_head(Q, K, V, dO, b, kept, full)
    eps = 1e-6
    for X, G in zip((Q, K, V), grads):
        for idx in np.ndindex(*X.shape):
            old = X[idx]
            X[idx] = old + eps
            lp = _loss(Q, K, V, dO, b, kept, full)
            X[idx] = old - eps
            lm = _loss(Q, K, V, dO, b, kept, full)
            X[idx] = old
            assert abs((lp - lm) / (2 * eps) - G[idx]) <= 1e-7, idx


def test_dense_limit_matches_torch_autograd():
    Ns, Nc, d, b = 24, 17, 8, 4
    Q, K, V, dO = _inputs(Ns, Nc, d, seed=11)
    kept, full = _plan(Q, K, V, b, 1.0, 1.0)
    dQ, dK, dV = bwd.oracle_backward_head(Q, K, V, dO, b, kept, full)
    q, k, v = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V))
    o = torch.nn.functional.scaled_dot_product_attention(q[None, None], k[None, None], v[None, None])[0, 0]
    o.backward(torch.tensor(dO))
    for mine, ref in ((dQ, q.grad), (dK, k.grad), (dV, v.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "Ns%d_Nc%d_d%d_b%d_r%g_g%g" % c)
def test_invariants(case):
    Ns, Nc, d, b, rho, gamma = case
    Q, K, V, dO = _inputs(Ns, Nc, d, seed=Ns + 5 * Nc)
    kept, full = _plan(Q, K, V, b, rho, gamma)
    dQ, dK, dV = bwd.oracle_backward_head(Q, K, V, dO, b, kept, full)
    # a common shift of every key leaves each softmax unchanged
    np.testing.assert_allclose(dK.sum(axis=0), 0.0, atol=1e-12)
    # a common shift of every value shifts every output by the same vector
    np.testing.assert_allclose(dV.sum(axis=0), dO.sum(axis=0), atol=1e-12)
    # Q -> cQ, K -> K/c leaves every logit unchanged
    assert abs((Q * dQ).sum() - (K * dK).sum()) <= 1e-11
    # pruned context rows take no part
    src, ctx = orc.block_ranges(Ns, Nc, b)
    for c, (s, e) in enumerate(ctx):
        if c not in set(int(x) for x in kept):
            assert not dK[s:e].any() and not dV[s:e].any()


def test_b1_is_independent_of_gamma():
    Ns, Nc, d, b = 9, 8, 3, 1
    Q, K, V, dO = _inputs(Ns, Nc, d, seed=21)
    kept, _ = _plan(Q, K, V, b, 0.5, 0.0)
    ref = bwd.oracle_backward_head(Q, K, V, dO, b, kept, np.arange(0))
    for kq in (3, Ns):
        full = np.arange(kq)
        got = bwd.oracle_backward_head(Q, K, V, dO, b, kept, full)
        for g, r in zip(got, ref):
            np.testing.assert_allclose(g, r, atol=1e-12)


def test_identical_keys_in_blocks_make_taylor_exact():
    Ns, Nc, d, b = 12, 9, 4, 3
    Q, K, V, dO = _inputs(Ns, Nc, d, seed=5)
    src, ctx = orc.block_ranges(Ns, Nc, b)
    for s, e in src + ctx:
        K[s:e] = K[s]
    kept, _ = _plan(Q, K, V, b, 0.5, 0.0)
    nb_s = len(src)
    t = bwd.oracle_backward_head(Q, K, V, dO, b, kept, np.arange(0))
    f = bwd.oracle_backward_head(Q, K, V, dO, b, kept, np.arange(nb_s))
    np.testing.assert_allclose(t[0], f[0], atol=1e-12)     # dQ
    np.testing.assert_allclose(t[2], f[2], atol=1e-12)     # dV: token weights are the block weight / n_j
    for s, e in src + ctx:                                   # dK: equal per block
        np.testing.assert_allclose(t[1][s:e].sum(axis=0), f[1][s:e].sum(axis=0), atol=1e-12)
