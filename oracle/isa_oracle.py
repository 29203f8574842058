"""Plain fp64 CPU oracle for In-context Sparse Attention (ISA).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.  It shares no
code with the HIP kernels.

What the method is
------------------
"Lightning Unified Video Editing via In-Context Sparse Attention"
(chatpaper.ai page), English abstract: in in-context video editing the
source-video tokens and the context (reference) tokens are concatenated and
attention over them is the bottleneck.  Context tokens carry much lower
saliency than source tokens, so a pre-selection step prunes redundant
context.  Query sharpness tracks the approximation error, so a dynamic query
grouping sends high-error queries to full attention and low-error ones to a
0-th order Taylor sparse attention.  The abstract names these steps and gives
no formula; the readings below fill them in.

Readings (the plainest ones the abstract supports)
--------------------------------------------------
R1  Queries are the Ns source rows.  Keys and values are the Ns source rows
    followed by the Nc context rows (the in-context concatenation).
R2  Blocks of b tokens partition each segment from its own start; the last
    block of a segment may be short.  Query blocks are the source blocks.
    Key-block order: source blocks, then context blocks.
R3  Block j has count n_j and the mean of its key rows (kbar_j) and value
    rows (vbar_j); pooled query qbar_i is the mean of block i's query rows.
R4  0-th order Taylor: expanding exp(q.k_t/sqrt d) around kbar_j and keeping
    the constant term, block j contributes n_j exp(q.kbar_j/sqrt d) with
    value vbar_j.
R5  Saliency of context block c: the probability that lands on c under the
    n-weighted pooled softmax of each pooled source query over ALL key
    blocks, summed (unweighted) over pooled source queries.
R6  Sharpness of query block i: the mean, over the block's queries, of the
    peak probability of the n-weighted pooled softmax over the kept key set.
R7  Count kept from n at fraction f: ceil(f*n - 1e-9) clipped to [0, n].
    Top-k by (score descending, index ascending); lists are ascending.
R8  Full route: exact softmax attention over every token of the kept key
    set (all source tokens and the tokens of the kept context blocks).
R9  Only context blocks are pruned; selection is per (batch, head).
N2  Context-token query rows (the other half of the in-context layer; the
    abstract defines pruning and grouping for the source queries only):
    ordinary attention of each context row over all Ns+Nc keys.

Special cases of the global self-attention formula used as pins are the
textbook form softmax(q k^T / sqrt(d_head)) v of "深度学习注意力机制：全局与
时间注意力的计算效率对比" (intelliparadigm.com), section 1 (global
self-attention).

Pins (tests/test_oracle_pins.py, tests/golden/)
-----------------------------------------------
* rho = gamma = 1 equals dense attention: torch CPU scaled_dot_product_attention
  in fp64 and a pure-Python loop over tokens.
* b = 1: Taylor equals full, output equals dense attention over source + kept
  context tokens for every gamma.
* keys identical inside each block: Taylor is exact, output independent of gamma.
* invariance to permuting tokens inside blocks; affine equivariance in V;
  scale invariance (cQ, K/c).
* saliency mass conservation: column sums over all key blocks total nb_s.
* K = 0 closed forms for sal, sh, the selected sets and O (ragged tails included).
* two hand-derived worked examples with exact fractions (tests/golden/).
* tie-break direction and routing direction on constructed inputs.
* the kept/routed counts of the five benchmark workloads (tests/golden/).
* an independent pure-Python loop implementation on tiny ragged shapes.
Parity unpinned: that R5, R6 and R7 are the exact choices of the paper's own
kernel.  The pages print no scores, sets or outputs for ISA, so these are
this project's definitions, pinned only by the properties above.
"""

import math

import numpy as np


def count_rule(f, n):
    """How many of n items a fraction f keeps (reading R7).

    The abstract says only that context is pruned and that a group of queries
    goes to full attention.  "Keep f" is read as "at least f": ceil(f*n),
    evaluated in fp64 with a 1e-9 guard so that products meant to be whole
    numbers are not pushed up by representation noise, clipped to [0, n].
    """
    f = float(f)
    n = int(n)
    return min(n, max(0, math.ceil(f * n - 1e-9)))


def block_ranges(Ns, Nc, b):
    """Row ranges of the source blocks and of the context blocks (R1, R2).

    Source rows are [0, Ns), context rows [Ns, Ns+Nc).  Each segment is cut
    into blocks of b rows from its own start; a block never spans both.
    """
    src = [(s, min(s + b, Ns)) for s in range(0, Ns, b)]
    ctx = [(Ns + s, Ns + min(s + b, Nc)) for s in range(0, Nc, b)]
    return src, ctx


def pool_blocks(X, ranges):
    """Per-block mean rows of X and per-block counts (R3)."""
    d = X.shape[1]
    if not ranges:
        return np.zeros((0, d)), np.zeros(0)
    means = np.stack([X[s:e].mean(axis=0) for s, e in ranges])
    counts = np.array([e - s for s, e in ranges], dtype=np.float64)
    return means, counts


def _weighted_softmax(logits, n):
    """Row-wise n_j exp(l_j) / sum_j' n_j' exp(l_j'), with max subtraction."""
    m = logits.max(axis=1, keepdims=True)
    w = n[None, :] * np.exp(logits - m)
    return w / w.sum(axis=1, keepdims=True)


def saliency_scores(qbar, kbar_all, n_all, nb_s, all_columns=False):
    """Context saliency (abstract: context tokens show much lower saliency
    than source tokens; reading R5).

    qbar: [nb_s, d] pooled source queries.  kbar_all, n_all: every key block,
    source first.  Returns sal[c] for the context blocks, or the column mass
    of every key block when all_columns is set.
    """
    d = qbar.shape[1]
    P = _weighted_softmax(qbar @ kbar_all.T / math.sqrt(d), n_all)
    col = P.sum(axis=0)
    return col if all_columns else col[nb_s:]


def top_indices(scores, k):
    """The k best indices by (score desc, index asc), returned ascending (R7)."""
    order = sorted(range(len(scores)), key=lambda j: (-float(scores[j]), j))
    return np.array(sorted(order[:k]), dtype=np.int64)


def sharpness_scores(Qs, src_ranges, kbar_K, n_K):
    """Query sharpness per source block (the abstract links a query's
    sharpness to the error of the approximate route; reading R6).

    Qs: [Ns, d] source queries.  kbar_K, n_K: the kept key blocks.
    sh_i = mean over q in block i of max_j P_j(q), P the n-weighted pooled
    softmax over the kept blocks.
    """
    d = Qs.shape[1]
    sh = np.empty(len(src_ranges))
    for i, (s, e) in enumerate(src_ranges):
        P = _weighted_softmax(Qs[s:e] @ kbar_K.T / math.sqrt(d), n_K)
        sh[i] = P.max(axis=1).mean()
    return sh


def full_attention_rows(q, Kt, Vt):
    """Exact softmax attention of the rows q over the tokens Kt, Vt (R8).

    The textbook global self-attention softmax(q k^T / sqrt d) v
    (intelliparadigm.com page, section 1), restricted to the given keys.
    """
    d = q.shape[1]
    logits = q @ Kt.T / math.sqrt(d)
    m = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - m)
    return (w @ Vt) / w.sum(axis=1, keepdims=True)


def taylor_attention_rows(q, kbar, vbar, n):
    """0-th order Taylor sparse attention over pooled blocks (abstract; R4).

    o = sum_j n_j exp(q.kbar_j/sqrt d) vbar_j / sum_j n_j exp(q.kbar_j/sqrt d).
    """
    d = q.shape[1]
    P = _weighted_softmax(q @ kbar.T / math.sqrt(d), n)
    return P @ vbar


def context_rows_forward(Qc, Kh, Vh):
    """Outputs of the context-token query rows (reading N2): every context row
    attends over all Ns+Nc keys, the textbook softmax(q k^T / sqrt d) v."""
    return full_attention_rows(_as64(Qc), _as64(Kh), _as64(Vh))


def dense_attention(Qh, Kh, Vh):
    """Dense attention of every query over every key (single head)."""
    return full_attention_rows(Qh, Kh, Vh)


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def oracle_plan_head(Qh, Kh, Vh, b, rho, gamma):
    """Selection half of ISA for one (batch, head).

    Qh: [Ns, d]; Kh, Vh: [Ns+Nc, d].  Returns a dict with the pooled blocks,
    sal, kept_ctx, sh, full_q and taylor_q (lists ascending, int64).
    """
    Qh, Kh, Vh = _as64(Qh), _as64(Kh), _as64(Vh)
    Ns = Qh.shape[0]
    Nc = Kh.shape[0] - Ns
    src, ctx = block_ranges(Ns, Nc, b)
    nb_s, nb_c = len(src), len(ctx)
    kbar_all, n_all = pool_blocks(Kh, src + ctx)
    vbar_all, _ = pool_blocks(Vh, src + ctx)
    qbar, _ = pool_blocks(Qh, src)
    sal = saliency_scores(qbar, kbar_all, n_all, nb_s)
    kc = count_rule(rho, nb_c)
    kept = top_indices(sal, kc)
    keyset = np.concatenate([np.arange(nb_s), nb_s + kept]).astype(np.int64)
    sh = sharpness_scores(Qh, src, kbar_all[keyset], n_all[keyset])
    kq = count_rule(gamma, nb_s)
    full_q = top_indices(sh, kq)
    taylor_q = np.array(sorted(set(range(nb_s)) - set(full_q.tolist())), dtype=np.int64)
    return {
        "nb_s": nb_s, "nb_c": nb_c, "kc": kc, "kq": kq,
        "qbar": qbar, "kbar": kbar_all, "vbar": vbar_all, "n": n_all,
        "sal": sal, "kept_ctx": kept, "keyset": keyset,
        "sh": sh, "full_q": full_q, "taylor_q": taylor_q,
    }


def oracle_forward_head(Qh, Kh, Vh, b, kept_ctx, full_q, rows=None):
    """Output half of ISA for one (batch, head), given the two index lists.

    Every source row is produced by exactly one route: rows of blocks in
    full_q by full attention over the tokens of the kept key set, the others
    by Taylor attention over the kept pooled blocks.  rows (optional) limits
    the work to those output rows; the result then has len(rows) rows.
    """
    Qh, Kh, Vh = _as64(Qh), _as64(Kh), _as64(Vh)
    Ns = Qh.shape[0]
    Nc = Kh.shape[0] - Ns
    src, ctx = block_ranges(Ns, Nc, b)
    nb_s = len(src)
    kept_ctx = [int(c) for c in kept_ctx]
    full = set(int(i) for i in full_q)
    kept_blocks = src + [ctx[c] for c in kept_ctx]
    kbar, n = pool_blocks(Kh, kept_blocks)
    vbar, _ = pool_blocks(Vh, kept_blocks)
    tok = np.concatenate([np.arange(s, e) for s, e in kept_blocks])
    Kt, Vt = Kh[tok], Vh[tok]
    want = np.arange(Ns) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((len(want), Qh.shape[1]))
    blk = want // b
    for i in range(nb_s):
        sel = np.nonzero(blk == i)[0]
        if sel.size == 0:
            continue
        q = Qh[want[sel]]
        if i in full:
            out[sel] = full_attention_rows(q, Kt, Vt)
        else:
            out[sel] = taylor_attention_rows(q, kbar, vbar, n)
    return out


def oracle_plan(Q, K, V, b, rho, gamma):
    """oracle_plan_head over every (batch, head) of [B, H, rows, d] arrays."""
    B, H = Q.shape[:2]
    heads = [[oracle_plan_head(Q[x, h], K[x, h], V[x, h], b, rho, gamma) for h in range(H)]
             for x in range(B)]
    out = {}
    for key in ("sal", "kept_ctx", "sh", "full_q", "taylor_q"):
        out[key] = np.stack([np.stack([heads[x][h][key] for h in range(H)]) for x in range(B)])
    for key in ("nb_s", "nb_c", "kc", "kq"):
        out[key] = heads[0][0][key]
    out["heads"] = heads
    return out


def oracle_forward(Q, K, V, b, kept_ctx, full_q):
    """oracle_forward_head over every (batch, head); lists shaped [B, H, k]."""
    B, H, Ns, d = Q.shape
    O = np.empty((B, H, Ns, d))
    for x in range(B):
        for h in range(H):
            O[x, h] = oracle_forward_head(Q[x, h], K[x, h], V[x, h], b, kept_ctx[x][h], full_q[x][h])
    return O


def isa_reference(Q, K, V, b, rho, gamma):
    """Whole ISA layer: (plan dict, O [B, H, Ns, d] fp64)."""
    plan = oracle_plan(Q, K, V, b, rho, gamma)
    O = oracle_forward(Q, K, V, b, plan["kept_ctx"], plan["full_q"])
    return plan, O
