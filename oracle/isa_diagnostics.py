"""Routing diagnostic for ISA on the CPU oracle (test infrastructure only).

"Lightning Unified Video Editing via In-Context Sparse Attention" (English
abstract) ties how sharp a query is to how badly the approximate route
serves it, which is why sharp query blocks go to full attention.  This
module measures that on synthetic inputs with the fp64 oracle alone:
  * the error of the 0-th order Taylor route per query block against the full
    route over the same kept key set (the block's error norm over the layer's
    output norm), and its Spearman rank correlation with the block sharpness
    sh_i;
  * the layer's relative error against all-full routing when the kq sharpest
    blocks take the full route (ISA), when kq random blocks do, and when the
    kq least sharp ones do (the inverse routing).

Run as `python -m oracle.isa_diagnostics` for the table over the within-block
locality sigma of sparse_attention_context_amd.synth.make_local_inputs.
"""

import numpy as np

from . import isa_oracle as orc


def _rank(x):
    order = np.argsort(x, kind="stable")
    r = np.empty(len(x))
    r[order] = np.arange(len(x))
    # average ranks of ties
    xs = np.asarray(x)[order]
    i = 0
    while i < len(xs):
        j = i
        while j + 1 < len(xs) and xs[j + 1] == xs[i]:
            j += 1
        r[order[i:j + 1]] = 0.5 * (i + j)
        i = j + 1
    return r


def spearman(x, y):
    """Spearman rank correlation: Pearson correlation of the (average) ranks."""
    rx, ry = _rank(x), _rank(y)
    rx, ry = rx - rx.mean(), ry - ry.mean()
    den = np.sqrt((rx * rx).sum() * (ry * ry).sum())
    return float((rx * ry).sum() / den) if den > 0 else 0.0


def routing_diagnostic(Qh, Kh, Vh, b, rho, gamma, seed=0, random_draws=4):
    """Per-block Taylor error and sharpness, and the layer error of three
    routings of kq blocks to the full route (sharpest, random, least sharp)."""
    p = orc.oracle_plan_head(Qh, Kh, Vh, b, rho, gamma)
    nb_s, kq, kept = p["nb_s"], p["kq"], p["kept_ctx"]
    Ns = Qh.shape[0]
    src, _ = orc.block_ranges(Ns, Kh.shape[0] - Ns, b)
    O_full = orc.oracle_forward_head(Qh, Kh, Vh, b, kept, np.arange(nb_s))
    O_tay = orc.oracle_forward_head(Qh, Kh, Vh, b, kept, np.arange(0))
    # each block's share of the layer error: its error norm over the layer's output norm
    err = np.array([np.linalg.norm(O_tay[s:e] - O_full[s:e]) for s, e in src]) / np.linalg.norm(O_full)

    def layer_err(full):
        O = orc.oracle_forward_head(Qh, Kh, Vh, b, kept, np.sort(np.asarray(full, dtype=np.int64)))
        return float(np.linalg.norm(O - O_full) / np.linalg.norm(O_full))

    order = sorted(range(nb_s), key=lambda j: (-float(p["sh"][j]), j))
    rng = np.random.default_rng(seed)
    return {
        "sh": p["sh"], "taylor_err": err, "spearman": spearman(p["sh"], err), "kq": kq,
        "layer_err_isa": layer_err(order[:kq]),
        "layer_err_inverse": layer_err(order[nb_s - kq:]),
        "layer_err_random": float(np.mean([layer_err(rng.permutation(nb_s)[:kq]) for _ in range(random_draws)])),
    }


def main():
    from sparse_attention_context_amd.synth import make_local_inputs
    Ns = Nc = 2048
    d, b, rho, gamma, H = 64, 64, 0.25, 0.2, 3
    print("Ns=Nc=%d d=%d b=%d rho=%g gamma=%g, %d heads per row" % (Ns, d, b, rho, gamma, H))
    print("%6s %10s %14s %12s %12s %12s" % ("sigma", "spearman", "taylor_err", "err_isa", "err_random", "err_inverse"))
    print("(taylor_err: layer error with every block on the Taylor route; err_*: layer error with kq blocks on the full route)")
    for sigma in (1.0, 0.5, 0.25, 0.1):
        Q, K, V = make_local_inputs(1, H, d, Ns, Nc, b, sigma, seed=11)
        rs = [routing_diagnostic(Q[0, h], K[0, h], V[0, h], b, rho, gamma, seed=h) for h in range(H)]
        print("%6.2f %10.3f %14.4f %12.4f %12.4f %12.4f" % (
            sigma, np.mean([r["spearman"] for r in rs]), np.mean([np.linalg.norm(r["taylor_err"]) for r in rs]),
            np.mean([r["layer_err_isa"] for r in rs]), np.mean([r["layer_err_random"] for r in rs]),
            np.mean([r["layer_err_inverse"] for r in rs])))


if __name__ == "__main__":
    main()
