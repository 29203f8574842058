"""Pins of the CPU oracle against facts it does not define itself.

Each test states what fixes the expected value: a hand-worked example, a
closed form, a library routine, an invariant of the definitions, or an
independent loop implementation.  No GPU is involved.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import isa_oracle as orc
from oracle.brute import brute_dense_head, brute_isa_head

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# fixture parsing

def _num(tok):
    if tok.endswith("*ln3"):
        return float(Fraction(tok[:-4])) * math.log(3.0)
    return float(Fraction(tok))


def _load_worked(name):
    params, rows = {}, {"Q": [], "K": [], "V": [], "O": []}
    lists = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            key = parts[0]
            if key == "param":
                params[parts[1]] = Fraction(parts[2])
            elif key in rows:
                rows[key].append([_num(t) for t in parts[1:]])
            else:
                lists[key] = [_num(t) for t in parts[1:]]
    return params, {k: np.array(v) for k, v in rows.items()}, lists


WORKED = ["worked_b1.txt", "worked_b2.txt", "worked_b2_gamma0.txt", "worked_ragged_k0.txt"]


@pytest.mark.parametrize("name", WORKED)
def test_worked_examples(name):
    p, r, lists = _load_worked(name)
    b = int(p["b"])
    plan = orc.oracle_plan_head(r["Q"], r["K"], r["V"], b, float(p["rho"]), float(p["gamma"]))
    np.testing.assert_allclose(plan["sal"], lists["sal"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(plan["sh"], lists["sh"], rtol=0, atol=1e-13)
    assert plan["kept_ctx"].tolist() == [int(x) for x in lists["kept_ctx"]]
    assert plan["full_q"].tolist() == [int(x) for x in lists["full_q"]]
    O = orc.oracle_forward_head(r["Q"], r["K"], r["V"], b, plan["kept_ctx"], plan["full_q"])
    np.testing.assert_allclose(O, r["O"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", WORKED)
def test_worked_examples_bruteforce(name):
    p, r, lists = _load_worked(name)
    kept, full, O = brute_isa_head(r["Q"].tolist(), r["K"].tolist(), r["V"].tolist(),
                                   int(p["b"]), float(p["rho"]), float(p["gamma"]))
    assert kept == [int(x) for x in lists["kept_ctx"]]
    assert full == [int(x) for x in lists["full_q"]]
    np.testing.assert_allclose(np.array(O), r["O"], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# count rule: the hand-derived table of the five workloads

def test_count_table():
    with open(os.path.join(GOLDEN, "counts.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 8
    for name, Ns, Nc, b, nb_s, nb_c, rho, kc, gamma, kq in rows:
        Ns, Nc, b = int(Ns), int(Nc), int(b)
        src, ctx = orc.block_ranges(Ns, Nc, b)
        assert len(src) == int(nb_s) and len(ctx) == int(nb_c), name
        assert orc.count_rule(float(rho), len(ctx)) == int(kc), name
        assert orc.count_rule(float(gamma), len(src)) == int(kq), name


def test_count_rule_edges():
    assert orc.count_rule(0.0, 10) == 0
    assert orc.count_rule(1.0, 10) == 10
    assert orc.count_rule(1e-12, 10) == 0      # below the guard
    assert orc.count_rule(0.01, 10) == 1       # any real fraction keeps one
    assert orc.count_rule(0.5, 0) == 0


# --------------------------------------------------------------------------
# helpers

def _rand(Ns, Nc, d, seed, kscale=1.0):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((Ns, d))
    K = rng.standard_normal((Ns + Nc, d)) * kscale
    V = rng.standard_normal((Ns + Nc, d))
    return Q, K, V


def _sdpa(q, K, V):
    """torch CPU scaled_dot_product_attention in fp64 (a library routine)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(K), t(V))[0, 0].numpy()


SHAPES = [  # (Ns, Nc, d, b)
    (37, 23, 8, 8),      # ragged source and context tails
    (64, 64, 16, 16),
    (50, 0, 8, 8),       # no context
    (9, 30, 4, 16),      # one source block (b >= Ns)
    (40, 25, 8, 1),      # b = 1
    (33, 70, 16, 7),
]


# --------------------------------------------------------------------------
# dense limit: rho = gamma = 1 is plain global attention

@pytest.mark.parametrize("Ns,Nc,d,b", SHAPES)
def test_dense_limit_matches_sdpa(Ns, Nc, d, b):
    Q, K, V = _rand(Ns, Nc, d, Ns * 7 + Nc)
    plan = orc.oracle_plan_head(Q, K, V, b, 1.0, 1.0)
    O = orc.oracle_forward_head(Q, K, V, b, plan["kept_ctx"], plan["full_q"])
    np.testing.assert_allclose(O, _sdpa(Q, K, V), rtol=0, atol=1e-12)


def test_dense_limit_matches_loop():
    Q, K, V = _rand(12, 9, 4, 3)
    plan = orc.oracle_plan_head(Q, K, V, 4, 1.0, 1.0)
    O = orc.oracle_forward_head(Q, K, V, 4, plan["kept_ctx"], plan["full_q"])
    ref = np.array(brute_dense_head(Q.tolist(), K.tolist(), V.tolist()))
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# b = 1: every block is a token, so the Taylor route is exact

@pytest.mark.parametrize("gamma", [0.0, 0.3, 1.0])
def test_b1_taylor_equals_full(gamma):
    Ns, Nc, d = 30, 40, 8
    Q, K, V = _rand(Ns, Nc, d, 11, kscale=0.7)
    plan = orc.oracle_plan_head(Q, K, V, 1, 0.4, gamma)
    O = orc.oracle_forward_head(Q, K, V, 1, plan["kept_ctx"], plan["full_q"])
    tok = np.concatenate([np.arange(Ns), Ns + plan["kept_ctx"]])
    np.testing.assert_allclose(O, _sdpa(Q, K[tok], V[tok]), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# identical keys inside every block: 0-th order Taylor is exact

def test_identical_keys_taylor_exact():
    Ns, Nc, d, b = 40, 36, 8, 8
    Q, K, V = _rand(Ns, Nc, d, 5)
    for s, e in sum(orc.block_ranges(Ns, Nc, b), []):
        K[s:e] = K[s]
    outs = []
    for gamma in (0.0, 0.5, 1.0):
        plan = orc.oracle_plan_head(Q, K, V, b, 0.5, gamma)
        outs.append(orc.oracle_forward_head(Q, K, V, b, plan["kept_ctx"], plan["full_q"]))
    np.testing.assert_allclose(outs[0], outs[2], rtol=0, atol=1e-12)
    np.testing.assert_allclose(outs[1], outs[2], rtol=0, atol=1e-12)
    tok = np.concatenate([np.arange(Ns)] + [np.arange(*orc.block_ranges(Ns, Nc, b)[1][c]) for c in plan["kept_ctx"]])
    np.testing.assert_allclose(outs[2], _sdpa(Q, K[tok], V[tok]), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# permutations inside blocks

def test_permutation_within_blocks():
    Ns, Nc, d, b = 37, 29, 8, 6
    Q, K, V = _rand(Ns, Nc, d, 21, kscale=0.8)
    base = orc.oracle_plan_head(Q, K, V, b, 0.5, 0.4)
    O = orc.oracle_forward_head(Q, K, V, b, base["kept_ctx"], base["full_q"])
    rng = np.random.default_rng(0)
    kperm = np.arange(Ns + Nc)
    qperm = np.arange(Ns)
    for s, e in sum(orc.block_ranges(Ns, Nc, b), []):
        kperm[s:e] = s + rng.permutation(e - s)
    for s, e in orc.block_ranges(Ns, Nc, b)[0]:
        qperm[s:e] = s + rng.permutation(e - s)
    plan = orc.oracle_plan_head(Q[qperm], K[kperm], V[kperm], b, 0.5, 0.4)
    assert plan["kept_ctx"].tolist() == base["kept_ctx"].tolist()
    assert plan["full_q"].tolist() == base["full_q"].tolist()
    np.testing.assert_allclose(plan["sal"], base["sal"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(plan["sh"], base["sh"], rtol=0, atol=1e-13)
    O2 = orc.oracle_forward_head(Q[qperm], K[kperm], V[kperm], b, plan["kept_ctx"], plan["full_q"])
    np.testing.assert_allclose(O2, O[qperm], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# affine equivariance in V, scale invariance, convexity

def test_affine_in_v():
    Ns, Nc, d, b = 33, 41, 8, 5
    Q, K, V = _rand(Ns, Nc, d, 8)
    p1 = orc.oracle_plan_head(Q, K, V, b, 0.3, 0.3)
    p2 = orc.oracle_plan_head(Q, K, 2.5 * V - 1.25, b, 0.3, 0.3)
    assert p1["kept_ctx"].tolist() == p2["kept_ctx"].tolist()
    assert p1["full_q"].tolist() == p2["full_q"].tolist()
    O1 = orc.oracle_forward_head(Q, K, V, b, p1["kept_ctx"], p1["full_q"])
    O2 = orc.oracle_forward_head(Q, K, 2.5 * V - 1.25, b, p1["kept_ctx"], p1["full_q"])
    np.testing.assert_allclose(O2, 2.5 * O1 - 1.25, rtol=0, atol=1e-12)


def test_scale_invariance():
    Ns, Nc, d, b = 40, 40, 8, 8
    Q, K, V = _rand(Ns, Nc, d, 9)
    p1 = orc.oracle_plan_head(Q, K, V, b, 0.5, 0.25)
    p2 = orc.oracle_plan_head(4.0 * Q, K / 4.0, V, b, 0.5, 0.25)
    assert p1["kept_ctx"].tolist() == p2["kept_ctx"].tolist()
    assert p1["full_q"].tolist() == p2["full_q"].tolist()
    O1 = orc.oracle_forward_head(Q, K, V, b, p1["kept_ctx"], p1["full_q"])
    O2 = orc.oracle_forward_head(4.0 * Q, K / 4.0, V, b, p2["kept_ctx"], p2["full_q"])
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-12)


def test_convexity():
    Ns, Nc, d, b = 64, 64, 8, 8
    Q, K, V = _rand(Ns, Nc, d, 10)
    plan = orc.oracle_plan_head(Q, K, V, b, 0.5, 0.5)
    O = orc.oracle_forward_head(Q, K, V, b, plan["kept_ctx"], plan["full_q"])
    src, ctx = orc.block_ranges(Ns, Nc, b)
    blocks = src + [ctx[c] for c in plan["kept_ctx"]]
    tok = np.concatenate([np.arange(s, e) for s, e in blocks])
    vbar, _ = orc.pool_blocks(V, blocks)
    for i, (s, e) in enumerate(src):
        if i in plan["full_q"]:
            lo, hi = V[tok].min(0), V[tok].max(0)
        else:
            lo, hi = vbar.min(0), vbar.max(0)
        assert np.all(O[s:e] >= lo - 1e-12) and np.all(O[s:e] <= hi + 1e-12)


# --------------------------------------------------------------------------
# saliency: probability mass is conserved over all key blocks

def test_saliency_conservation():
    Ns, Nc, d, b = 45, 77, 8, 8
    Q, K, V = _rand(Ns, Nc, d, 12)
    src, ctx = orc.block_ranges(Ns, Nc, b)
    kbar, n = orc.pool_blocks(K, src + ctx)
    qbar, _ = orc.pool_blocks(Q, src)
    col = orc.saliency_scores(qbar, kbar, n, len(src), all_columns=True)
    assert abs(col.sum() - len(src)) < 1e-12
    sal = orc.saliency_scores(qbar, kbar, n, len(src))
    np.testing.assert_allclose(sal, col[len(src):], rtol=0, atol=0)


# --------------------------------------------------------------------------
# K = 0: closed forms for every score, set and output

@pytest.mark.parametrize("Ns,Nc,b,rho,gamma", [(48, 40, 8, 0.5, 0.25), (45, 37, 8, 0.4, 0.5), (20, 11, 4, 1.0, 0.0)])
def test_zero_keys_closed_form(Ns, Nc, b, rho, gamma):
    d = 8
    Q, _, V = _rand(Ns, Nc, d, 13)
    K = np.zeros((Ns + Nc, d))
    src, ctx = orc.block_ranges(Ns, Nc, b)
    n_src = np.array([e - s for s, e in src], float)
    n_ctx = np.array([e - s for s, e in ctx], float)
    plan = orc.oracle_plan_head(Q, K, V, b, rho, gamma)
    total = n_src.sum() + n_ctx.sum()
    np.testing.assert_allclose(plan["sal"], len(src) * n_ctx / total, rtol=0, atol=1e-13)
    kc = orc.count_rule(rho, len(ctx))
    # larger blocks first, ties to the lower index
    expect_kept = sorted(sorted(range(len(ctx)), key=lambda c: (-n_ctx[c], c))[:kc])
    assert plan["kept_ctx"].tolist() == expect_kept
    nk = np.concatenate([n_src, n_ctx[expect_kept]])
    np.testing.assert_allclose(plan["sh"], np.full(len(src), nk.max() / nk.sum()), rtol=0, atol=1e-13)
    assert plan["full_q"].tolist() == list(range(orc.count_rule(gamma, len(src))))
    O = orc.oracle_forward_head(Q, K, V, b, plan["kept_ctx"], plan["full_q"])
    tok = np.concatenate([np.arange(Ns)] + [np.arange(*ctx[c]) for c in expect_kept])
    np.testing.assert_allclose(O, np.broadcast_to(V[tok].mean(0), O.shape), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# direction of the two selections and the tie rule

def test_salient_context_block_is_kept_and_ties_go_low():
    Ns, Nc, d, b = 32, 64, 8, 8
    rng = np.random.default_rng(3)
    Q = rng.standard_normal((Ns, d))
    K = np.zeros((Ns + Nc, d))
    K[:Ns] = rng.standard_normal((Ns, d))
    qbar = Q.mean(0)
    K[Ns + 5 * b:Ns + 6 * b] = 3.0 * qbar / np.linalg.norm(qbar)   # block 5 aligned with queries
    V = rng.standard_normal((Ns + Nc, d))
    plan = orc.oracle_plan_head(Q, K, V, b, 0.25, 0.5)   # keep 2 of 8
    assert plan["kept_ctx"].tolist() == [0, 5]


def test_sharp_block_routed_to_full():
    Ns, Nc, d, b = 64, 64, 16, 8
    rng = np.random.default_rng(4)
    Q = 0.1 * rng.standard_normal((Ns, d))
    K = rng.standard_normal((Ns + Nc, d))
    Q[3 * b:4 * b] = 6.0 * K[10]          # block 3 queries point at one source block
    V = rng.standard_normal((Ns + Nc, d))
    plan = orc.oracle_plan_head(Q, K, V, b, 0.5, 0.125)   # one block to full
    assert plan["full_q"].tolist() == [3]
    assert plan["sh"][3] == plan["sh"].max()


def test_top_indices_tie_rule():
    s = np.array([0.5, 0.9, 0.5, 0.9, 0.1, 0.5])
    assert orc.top_indices(s, 3).tolist() == [0, 1, 3]
    assert orc.top_indices(s, 0).tolist() == []
    assert orc.top_indices(s, 6).tolist() == list(range(6))


# --------------------------------------------------------------------------
# vectorised oracle vs the independent loop implementation

@pytest.mark.parametrize("Ns,Nc,d,b,rho,gamma", [
    (37, 23, 4, 8, 0.5, 0.4),
    (20, 0, 4, 4, 0.5, 0.5),
    (9, 30, 4, 16, 0.3, 1.0),
    (24, 18, 3, 1, 0.4, 0.2),
    (33, 41, 6, 5, 0.0, 0.6),
    (28, 28, 4, 7, 1.0, 0.0),
])
def test_against_loop_implementation(Ns, Nc, d, b, rho, gamma):
    Q, K, V = _rand(Ns, Nc, d, Ns + 3 * Nc + d, kscale=0.8)
    Q[: Ns // 4] += 3.0 * K[: Ns // 4]
    plan = orc.oracle_plan_head(Q, K, V, b, rho, gamma)
    O = orc.oracle_forward_head(Q, K, V, b, plan["kept_ctx"], plan["full_q"])
    kept, full, Ob = brute_isa_head(Q.tolist(), K.tolist(), V.tolist(), b, rho, gamma)
    assert plan["kept_ctx"].tolist() == kept
    assert plan["full_q"].tolist() == full
    np.testing.assert_allclose(O, np.array(Ob), rtol=0, atol=1e-12)


def test_forward_rows_subset():
    Ns, Nc, d, b = 50, 30, 8, 8
    Q, K, V = _rand(Ns, Nc, d, 31)
    plan = orc.oracle_plan_head(Q, K, V, b, 0.5, 0.5)
    O = orc.oracle_forward_head(Q, K, V, b, plan["kept_ctx"], plan["full_q"])
    rows = [49, 0, 17, 8, 8, 33]
    Or = orc.oracle_forward_head(Q, K, V, b, plan["kept_ctx"], plan["full_q"], rows=rows)
    np.testing.assert_allclose(Or, O[rows], rtol=0, atol=1e-14)


def test_batched_entry_points():
    rng = np.random.default_rng(2)
    Q = rng.standard_normal((2, 3, 20, 4))
    K = rng.standard_normal((2, 3, 35, 4))
    V = rng.standard_normal((2, 3, 35, 4))
    plan, O = orc.isa_reference(Q, K, V, 4, 0.5, 0.5)
    for x in range(2):
        for h in range(3):
            ph = orc.oracle_plan_head(Q[x, h], K[x, h], V[x, h], 4, 0.5, 0.5)
            assert plan["kept_ctx"][x, h].tolist() == ph["kept_ctx"].tolist()
            assert plan["full_q"][x, h].tolist() == ph["full_q"].tolist()
            Oh = orc.oracle_forward_head(Q[x, h], K[x, h], V[x, h], 4, ph["kept_ctx"], ph["full_q"])
            np.testing.assert_allclose(O[x, h], Oh, rtol=0, atol=1e-14)


def test_context_rows_match_torch_sdpa():
    # reading N2: context queries attend over every key, as plain attention does
    rng = np.random.default_rng(17)
    Qc, K, V = rng.standard_normal((23, 8)), rng.standard_normal((40, 8)), rng.standard_normal((40, 8))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(Qc)[None, None], torch.tensor(K)[None, None], torch.tensor(V)[None, None])[0, 0].numpy()
    np.testing.assert_allclose(orc.context_rows_forward(Qc, K, V), ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(orc.context_rows_forward(Qc, K, V), brute_dense_head(Qc, K, V), rtol=0, atol=1e-12)
