"""Pure-Python loop implementation of ISA for tiny inputs -- TEST INFRASTRUCTURE.

A second, independent writing of the definitions in ``isa_oracle`` (the
readings R1-R9 listed there), token by token with ``math.exp`` and Python
lists, no NumPy.  It exists only to cross-check the vectorised oracle on
shapes small enough for loops (tens of tokens, d of a few units).

Method: "Lightning Unified Video Editing via In-Context Sparse Attention"
(chatpaper.ai page), English abstract -- context pre-selection, query
grouping by sharpness, full attention for high-error queries and 0-th order
Taylor sparse attention for the rest.
"""

import math


def _dot(a, b):
    s = 0.0
    for x, y in zip(a, b):
        s += x * y
    return s


def _mean_rows(rows):
    n = len(rows)
    d = len(rows[0])
    return [sum(r[c] for r in rows) / n for c in range(d)]


def _blocks(lo, hi, b):
    out = []
    s = lo
    while s < hi:
        out.append(list(range(s, min(s + b, hi))))
        s += b
    return out


def _probs(q, keys, weights, d):
    """weights[j] * exp(q.keys[j]/sqrt d), normalised; explicit max shift."""
    lg = [_dot(q, k) / math.sqrt(d) for k in keys]
    m = max(lg)
    w = [weights[j] * math.exp(lg[j] - m) for j in range(len(keys))]
    tot = sum(w)
    return [x / tot for x in w]


def _kept_count(f, n):
    c = math.ceil(f * n - 1e-9)
    return min(n, max(0, c))


def _best(scores, k):
    idx = list(range(len(scores)))
    # selection by repeated arg-max: the highest score, lowest index first
    chosen = []
    for _ in range(k):
        best = None
        for j in idx:
            if j in chosen:
                continue
            if best is None or scores[j] > scores[best]:
                best = j
        chosen.append(best)
    return sorted(chosen)


def brute_isa_head(Q, K, V, b, rho, gamma):
    """ISA on one head given as lists of rows.  Returns (kept, full, O)."""
    Ns = len(Q)
    Nc = len(K) - Ns
    d = len(Q[0])
    sblk = _blocks(0, Ns, b)
    cblk = _blocks(Ns, Ns + Nc, b)
    allblk = sblk + cblk
    kbar = [_mean_rows([K[t] for t in blk]) for blk in allblk]
    vbar = [_mean_rows([V[t] for t in blk]) for blk in allblk]
    cnt = [float(len(blk)) for blk in allblk]
    qbar = [_mean_rows([Q[t] for t in blk]) for blk in sblk]

    sal = [0.0] * len(cblk)
    for qb in qbar:
        p = _probs(qb, kbar, cnt, d)
        for c in range(len(cblk)):
            sal[c] += p[len(sblk) + c]
    kept = _best(sal, _kept_count(rho, len(cblk)))

    kidx = list(range(len(sblk))) + [len(sblk) + c for c in kept]
    kk = [kbar[j] for j in kidx]
    kv = [vbar[j] for j in kidx]
    kn = [cnt[j] for j in kidx]

    sh = []
    for blk in sblk:
        peaks = [max(_probs(Q[t], kk, kn, d)) for t in blk]
        sh.append(sum(peaks) / len(peaks))
    full = _best(sh, _kept_count(gamma, len(sblk)))

    toks = [t for j in kidx for t in allblk[j]]
    O = []
    for i, blk in enumerate(sblk):
        for t in blk:
            q = Q[t]
            if i in full:
                p = _probs(q, [K[u] for u in toks], [1.0] * len(toks), d)
                O.append([sum(p[a] * V[toks[a]][c] for a in range(len(toks))) for c in range(d)])
            else:
                p = _probs(q, kk, kn, d)
                O.append([sum(p[a] * kv[a][c] for a in range(len(kk))) for c in range(d)])
    return kept, full, O


def brute_dense_head(Q, K, V):
    """softmax(q k^T / sqrt d) v for every query row, by loops."""
    d = len(Q[0])
    O = []
    for q in Q:
        p = _probs(q, K, [1.0] * len(K), d)
        O.append([sum(p[a] * V[a][c] for a in range(len(K))) for c in range(d)])
    return O
