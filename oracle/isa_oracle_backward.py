"""Plain fp64 CPU oracle for the backward pass of In-context Sparse Attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.  It shares no
code with the HIP kernels.

What is differentiated
----------------------
The forward of "Lightning Unified Video Editing via In-Context Sparse
Attention" (chatpaper.ai page, English abstract), read as in isa_oracle.py:
full-route rows attend exactly over the tokens of the kept key set (R8),
Taylor rows attend over the kept pooled blocks with weights n_j (R4).  The
pages give no backward pass; the gradients below are the derivatives of
those forward definitions, with these readings:

B1  The plan is frozen: kept_ctx and full_q are discrete decisions taken by
    the selection half and are constants of the backward pass.  Saliency and
    sharpness receive no gradient.
B2  The block counts n_j are constants.
B3  A pooled key (value) is the mean of its block's rows, so its gradient is
    shared equally: dk_t += dkbar_j / n_j for every row t of block j.
B4  Rows that take part in neither route (the rows of pruned context blocks)
    get zero gradient.

With L = sum(dO * O) and, for a softmax row p = softmax(l):
    D_i = dO_i . o_i,   dl_ij = p_ij (dO_i . v_j - D_i),
    dq_i = sum_j dl_ij k_j / sqrt d,  dk_j = sum_i dl_ij q_i / sqrt d,
    dv_j = sum_i p_ij dO_i,
the n_j weights of the Taylor route entering p only as constants (B2).

Pins (tests/test_oracle_backward_pins.py): central finite differences of the
forward oracle along random directions and element by element on tiny ragged
shapes; the dense limit against torch fp64 autograd of
scaled_dot_product_attention; sum_t dK_t = 0 (softmax is blind to a common
shift of the keys), sum_t dV_t = sum_i dO_i (the weights of a row sum to 1),
sum Q*dQ = sum K*dK (invariance under Q -> cQ, K -> K/c); b = 1 independent of
gamma; keys identical inside blocks (Taylor exact) give the same dQ and dV
for every gamma; zero gradient on pruned context rows.
"""

import math

import numpy as np

from .isa_oracle import block_ranges, pool_blocks


def _softmax_rows(logits, n=None):
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    if n is not None:
        w = w * n[None, :]
    return w / w.sum(axis=1, keepdims=True)


def full_attention_rows_backward(q, Kt, Vt, dO):
    """Gradients of the exact attention of rows q over tokens Kt, Vt (R8).

    Returns (dq, dKt, dVt) for the upstream gradient dO of the outputs.
    """
    d = q.shape[1]
    P = _softmax_rows(q @ Kt.T / math.sqrt(d))
    O = P @ Vt
    D = (dO * O).sum(axis=1, keepdims=True)
    dL = P * (dO @ Vt.T - D)
    dq = dL @ Kt / math.sqrt(d)
    dKt = dL.T @ q / math.sqrt(d)
    dVt = P.T @ dO
    return dq, dKt, dVt


def taylor_attention_rows_backward(q, kbar, vbar, n, dO):
    """Gradients of the 0-th order Taylor attention over pooled blocks (R4, B2).

    Returns (dq, dkbar, dvbar): gradients with respect to the queries and to
    the pooled keys and values (not yet spread over the block rows).
    """
    d = q.shape[1]
    P = _softmax_rows(q @ kbar.T / math.sqrt(d), n)
    O = P @ vbar
    D = (dO * O).sum(axis=1, keepdims=True)
    dL = P * (dO @ vbar.T - D)
    dq = dL @ kbar / math.sqrt(d)
    dkbar = dL.T @ q / math.sqrt(d)
    dvbar = P.T @ dO
    return dq, dkbar, dvbar


def oracle_backward_head(Qh, Kh, Vh, dOh, b, kept_ctx, full_q):
    """dQ [Ns, d], dK and dV [Ns+Nc, d] of one (batch, head), plan frozen (B1).

    Full-route rows contribute through the kept tokens, Taylor rows through
    the kept pooled blocks; pooled gradients are spread over the block rows
    (B3); pruned context rows stay zero (B4).
    """
    Qh, Kh, Vh, dOh = (np.asarray(x, dtype=np.float64) for x in (Qh, Kh, Vh, dOh))
    Ns = Qh.shape[0]
    Nc = Kh.shape[0] - Ns
    src, ctx = block_ranges(Ns, Nc, b)
    nb_s = len(src)
    kept_blocks = src + [ctx[int(c)] for c in kept_ctx]
    tok = np.concatenate([np.arange(s, e) for s, e in kept_blocks]) if kept_blocks else np.zeros(0, np.int64)
    full = set(int(i) for i in full_q)
    full_rows = np.concatenate([np.arange(*src[i]) for i in range(nb_s) if i in full] or [np.zeros(0, np.int64)])
    tay_rows = np.concatenate([np.arange(*src[i]) for i in range(nb_s) if i not in full] or [np.zeros(0, np.int64)])

    dQ = np.zeros_like(Qh)
    dK = np.zeros_like(Kh)
    dV = np.zeros_like(Vh)
    if full_rows.size:
        dq, dKt, dVt = full_attention_rows_backward(Qh[full_rows], Kh[tok], Vh[tok], dOh[full_rows])
        dQ[full_rows] = dq
        dK[tok] += dKt
        dV[tok] += dVt
    if tay_rows.size:
        kbar, n = pool_blocks(Kh, kept_blocks)
        vbar, _ = pool_blocks(Vh, kept_blocks)
        dq, dkbar, dvbar = taylor_attention_rows_backward(Qh[tay_rows], kbar, vbar, n, dOh[tay_rows])
        dQ[tay_rows] = dq
        for j, (s, e) in enumerate(kept_blocks):
            dK[s:e] += dkbar[j] / n[j]
            dV[s:e] += dvbar[j] / n[j]
    return dQ, dK, dV


def oracle_backward(Q, K, V, dO, b, kept_ctx, full_q):
    """oracle_backward_head over every (batch, head) of [B, H, rows, d] arrays."""
    B, H = Q.shape[:2]
    dQ = np.zeros(Q.shape)
    dK = np.zeros(K.shape)
    dV = np.zeros(V.shape)
    for x in range(B):
        for h in range(H):
            dQ[x, h], dK[x, h], dV[x, h] = oracle_backward_head(Q[x, h], K[x, h], V[x, h], dO[x, h], b,
                                                                kept_ctx[x][h], full_q[x][h])
    return dQ, dK, dV
