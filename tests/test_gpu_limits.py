"""GPU parity at the largest head count the library accepts, B*H = 65535.

Several launches put B*H on grid y (the saliency pass, the backward's
pruned-row zeroing), or run one workgroup per head on grid x (the two
selections), and the persistent kernels deal heads out in turn, so the last
heads are where an indexing or grid limit would show.  The heads are tiny
(a few rows, ragged blocks), so the check is cheap per head: a fixed sample
of about 1700 heads -- the first and last 512 and every 97th one -- is
compared with the oracle as in test_gpu_parity (pooled means, scores, index
sets, every output row), and every head's output must be finite and inside
the range of its value rows (each output row is a convex combination of
them, up to bf16 rounding).  Pooled vectors of two or three tokens with
sharp queries are long, so the bf16 hi + lo representation of the pooled
operands moves saliency and sharpness by up to a few 1e-6 here: both
tolerances, and the bands of the two set checks, widen to the bounds of
_saliency_bound and _sharpness_bound where those exceed 1e-6 (recorded)."""

import numpy as np
import pytest
import torch

from oracle import isa_oracle as orc
from oracle import isa_oracle_backward as bwd
from sparse_attention_context_amd import isa
from sparse_attention_context_amd.synth import make_inputs, make_inputs_device, round_to_bf16
from tests.parity_util import assert_output, check_set, device_tensor
from tests.test_gpu_backward import GRAD_MAXREL, GRAD_RELL2, _grad_errors
from tests.test_gpu_parity import _host_views, _plan_checks

pytestmark = pytest.mark.gpu

MAX_BH = 65535


def _sample_heads(n):
    return sorted(set(range(min(512, n))) | set(range(max(0, n - 512), n)) | set(range(0, n, 97)))


def _in_value_range(O, V):
    """O [heads, rows, d], V [heads, keys, d]: every output entry lies within
    [min, max] of its head's value column (plus bf16 slack)."""
    lo = V.min(axis=1, keepdims=True)   # [heads, 1, d]
    hi = V.max(axis=1, keepdims=True)
    slack = 2.0 ** -7 * np.maximum(np.abs(lo), np.abs(hi)) + 1e-6
    return bool(np.all(np.isfinite(O)) and np.all(O >= lo - slack) and np.all(O <= hi + slack))


CASES = [
    # B, H, d, Ns, Nc, b, rho, gamma
    (3, 21845, 64, 5, 3, 2, 0.5, 0.5),
    (1, 65535, 128, 7, 5, 3, 0.5, 0.4),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dd%d_Ns%d_Nc%d_b%d_r%g_g%g" % c)
def test_most_heads_forward(case, parity_record):
    B, H, d, Ns, Nc, b, rho, gamma = case
    assert B * H == MAX_BH
    print("heads limit case %s" % (case,), flush=True)
    Q, K, V = make_inputs(B, H, d, Ns, Nc, seed=Ns + Nc + d, dtype="bf16")
    Qd, Kd, Vd = (device_tensor(t, "bf16") for t in (Q, K, V))
    O, ws = isa.attention(Qd, Kd, Vd, b, rho, gamma)
    torch.cuda.synchronize()
    Oh = O.float().cpu().numpy()
    assert _in_value_range(Oh.reshape(B * H, Ns, d), V.reshape(B * H, Ns + Nc, d))
    hv = _host_views(isa.plan_views(Qd, Kd, ws, b, rho, gamma))
    rec = {"case": "heads limit B%dH%dd%d_Ns%d_Nc%d_b%d" % (B, H, d, Ns, Nc, b), "maxabs": 0.0, "rel_l2": 0.0,
           "max_sal_err": 0.0, "max_sh_err": 0.0, "sal_bound": 0.0, "sh_bound": 0.0, "ambiguous_ctx": 0,
           "ambiguous_q": 0, "heads_compared": 0}
    heads = _sample_heads(B * H)
    for i, g in enumerate(heads):
        x, h = divmod(g, H)
        st, kept, full = _plan_checks(Q[x, h], K[x, h], V[x, h], b, rho, gamma, hv, x, h, sh_bound=True,
                                      sal_bound=True)
        Oref = orc.oracle_forward_head(Q[x, h], K[x, h], V[x, h], b, kept, full)
        maxabs, rel = assert_output(Oh[x, h], Oref, "bf16")
        rec["maxabs"] = max(rec["maxabs"], maxabs)
        rec["rel_l2"] = max(rec["rel_l2"], rel)
        rec["max_sal_err"] = max(rec["max_sal_err"], st["sal_err"])
        rec["max_sh_err"] = max(rec["max_sh_err"], st["sh_err"])
        rec["sal_bound"] = max(rec["sal_bound"], st.get("sal_bound", 0.0))
        rec["sh_bound"] = max(rec["sh_bound"], st.get("sh_bound", 0.0))
        rec["ambiguous_ctx"] += st["amb_ctx"]
        rec["ambiguous_q"] += st["amb_q"]
        if i % 500 == 499:
            print("  %d heads compared" % (i + 1), flush=True)
    rec["heads_compared"] = len(heads)
    parity_record(rec)


def test_most_heads_backward():
    B, H, d, Ns, Nc, b, rho, gamma = 1, MAX_BH, 128, 7, 5, 3, 0.5, 0.4
    print("heads limit backward", flush=True)
    Q, K, V = make_inputs(B, H, d, Ns, Nc, seed=77, dtype="bf16")
    dO = round_to_bf16(np.random.default_rng(78).standard_normal((B, H, Ns, d)).astype(np.float32))
    Qd, Kd, Vd, dOd = (device_tensor(t, "bf16") for t in (Q, K, V, dO))
    O, ws = isa.attention(Qd, Kd, Vd, b, rho, gamma)
    dQ, dK, dV, _ = isa.backward(Qd, Kd, Vd, O, dOd, ws, b, rho, gamma)
    torch.cuda.synchronize()
    views = isa.plan_views(Qd, Kd, ws, b, rho, gamma)
    kept = views["kept_ctx"].cpu().numpy()
    full = views["full_q"].cpu().numpy()
    heads = _sample_heads(H)
    got = [g.float().cpu().numpy()[0, heads] for g in (dQ, dK, dV)]
    assert all(np.all(np.isfinite(g)) for g in got)
    ref = [np.zeros_like(g, dtype=np.float64) for g in got]
    for i, h in enumerate(heads):
        r = bwd.oracle_backward_head(Q[0, h], K[0, h], V[0, h], dO[0, h], b, kept[0, h], full[0, h])
        for t in range(3):
            ref[t][i] = r[t]
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        maxrel, rel = _grad_errors(g, r)
        print("  %s max/scale %.2e rel-L2 %.2e over %d heads" % (name, maxrel, rel, len(heads)), flush=True)
        assert maxrel <= GRAD_MAXREL and rel <= GRAD_RELL2, (name, maxrel, rel)


SPAN_CASES = [
    # d, Ns, Nc, rho, gamma: K and V span just under 2^31 bytes per head
    (128, 4194000, 4194300, 0.25, 0.002),
    (64, 8388000, 8389215, 0.25, 0.001),    # also the largest row count, Ns + Nc = 2^24 - 1
]


@pytest.mark.parametrize("case", SPAN_CASES, ids=lambda c: "d%d_Ns%d_Nc%d" % c[:3])
def test_largest_head_span(case, parity_record):
    """One head whose K and V each span just under 2^31 bytes, the most the
    kernels' 32-bit offsets address (at d = 64 also the largest row count
    the library accepts), b = 256 with ragged last blocks on both sides, a
    quarter of the context kept and 33 query blocks on the full route, each
    over millions of keys.  The oracle checks what it can at this size:
    every pooled query and key mean, every saliency score (the oracle run on
    chunks of the pooled queries, whose column sums add up) and the kept
    set; the sharpness of 16 blocks (the first, the last, the full route's
    first and last, and spread ones); the query set as the top-k of the GPU's
    own scores under the tie rule; and 264 output rows (two of each of four
    full blocks, 256 Taylor rows), element by element."""
    d, Ns, Nc, rho, gamma = case
    B, H, b = 1, 1, 256
    assert Ns + Nc < 1 << 24 and (Ns + Nc) * d * 2 < 1 << 31 <= (Ns + Nc + 8192) * d * 2
    print("largest head span: d %d Ns %d Nc %d" % (d, Ns, Nc), flush=True)
    dev = torch.device("cuda:0")
    Qd, Kd, Vd = make_inputs_device(B, H, d, Ns, Nc, 4242 + d, dev, "bf16")
    O, ws = isa.attention(Qd, Kd, Vd, b, rho, gamma)
    torch.cuda.synchronize()
    hv = _host_views(isa.plan_views(Qd, Kd, ws, b, rho, gamma))
    Q = Qd[0, 0].double().cpu().numpy()
    K = Kd[0, 0].double().cpu().numpy()
    V = Vd[0, 0].double().cpu().numpy()
    Oh = O[0, 0].float().cpu().numpy()
    del Qd, Kd, Vd, O, ws
    torch.cuda.empty_cache()
    print("  layer ran; oracle pooling", flush=True)
    src, ctx = orc.block_ranges(Ns, Nc, b)
    nb_s, nb_c = len(src), len(ctx)
    kc, kq = orc.count_rule(rho, nb_c), orc.count_rule(gamma, nb_s)
    qbar, _ = orc.pool_blocks(Q, src)
    kbar, n = orc.pool_blocks(K, src + ctx)
    kept = hv["kept_ctx"][0, 0]
    full = hv["full_q"][0, 0]
    assert len(kept) == kc and len(full) == kq
    have = list(range(nb_s)) + [nb_s + int(c) for c in kept]
    vbar, _ = orc.pool_blocks(V, [(src + ctx)[j] for j in have])
    pool_err = max(float(np.abs(hv["qbar"][0, 0] - qbar).max()), float(np.abs(hv["kbar"][0, 0] - kbar).max()),
                   float(np.abs(hv["vbar"][0, 0][have] - vbar).max()))
    assert pool_err <= 2e-6, pool_err
    print("  saliency", flush=True)
    sal = sum(orc.saliency_scores(qbar[i:i + 4096], kbar, n, nb_s) for i in range(0, nb_s, 4096))
    sal_err = float(np.abs(hv["sal"][0, 0] - sal).max())
    assert sal_err < 1e-6, sal_err
    amb_ctx = check_set(kept, sal, kc)
    print("  sharpness of sampled blocks", flush=True)
    keyset = np.concatenate([np.arange(nb_s), nb_s + kept.astype(np.int64)])
    blocks = sorted({0, nb_s - 1, int(full[0]), int(full[-1])} | set(range(0, nb_s, nb_s // 12)))
    sh_ref = orc.sharpness_scores(Q, [src[i] for i in blocks], kbar[keyset], n[keyset])
    sh = hv["sh"][0, 0]
    sh_err = float(np.abs(sh[blocks] - sh_ref).max())
    assert sh_err < 1e-6, sh_err
    # the query set is the top-kq of the GPU's own scores, ties to the lower index
    assert full.tolist() == orc.top_indices(sh, kq).tolist()
    tayl = hv["taylor_q"][0, 0]
    assert sorted(set(full.tolist()) | set(tayl.tolist())) == list(range(nb_s))
    print("  sampled output rows", flush=True)
    rng = np.random.default_rng(5)
    rows = set()
    for i in (int(full[0]), int(full[1]), int(full[-2]), int(full[-1])):
        s, e = src[i]
        rows |= {s, e - 1}
    taylor_rows = np.concatenate([np.arange(s, e) for s, e in (src[int(t)] for t in tayl[:: max(1, len(tayl) // 64)])])
    rows |= set(rng.choice(taylor_rows, 255, replace=False).tolist()) | {Ns - 1}
    rows = np.array(sorted(rows))
    Oref = orc.oracle_forward_head(Q, K, V, b, kept, full, rows=rows)
    maxabs, rel = assert_output(Oh[rows], Oref, "bf16")
    parity_record({"case": "largest head span d %d Ns %d Nc %d b %d" % (d, Ns, Nc, b), "maxabs": maxabs,
                   "rel_l2": rel, "max_pool_err": pool_err, "max_sal_err": sal_err, "max_sh_err": sh_err,
                   "ambiguous_ctx": amb_ctx, "rows_compared": int(rows.size), "sh_blocks_compared": len(blocks)})


@pytest.mark.parametrize("case", SPAN_CASES, ids=lambda c: "d%d_Ns%d_Nc%d" % c[:3])
def test_largest_head_span_backward(case):
    """The backward pass on the largest head span (the shapes above).

    Rows of pruned context blocks must be exactly zero, and two sums that
    hold at any size are checked per feature c in fp64:
      sum_t dV_t = sum_i dO_i: the kernels round p to bf16 before dV = p^T dO
        (a row's weights then sum to 1 within 2^-9) and round dV to bf16, so
        |sum_t dV_tc - sum_i dO_ic| <= 2^-9 (sum_i |dO_ic| + sum_t |dV_tc|);
      sum_t dK_t = 0: with ds_it = p_it (dP_it - D_i), sum_t ds_it vanishes
        up to the bf16 rounding of ds (2^-9 of sum_t |ds_it| <= 2 max_t |dP_it|
        <= 2 |dO_i|_1 max|V|) and of the output in D_i (2^-9 |o_i| |dO_i|_1), so
        |sum_t dK_tc| <= 2^-9 sum_t |dK_tc| + 2^-7 max|V| sum_i |dO_i|_1 |q_ic| / sqrt d.
    (Both are worst-case bounds of the roundings; the measured sums sit far
    inside them and are printed.)

    dQ of 264 sampled rows (8 full-route rows over all 5.2 M or 10.5 M kept
    tokens, 256 Taylor rows) against the oracle's row gradients.  The
    kernels take D_i = dO_i . o_i from the layer's bf16 output, as flash
    attention does; the oracle takes it from the exact output.  Since dq_i
    is linear in D_i (dq_i = sum_t p_it (dP_it - D_i) k_t / sqrt d), the
    oracle's gradient is moved by -(D~_i - D_i) kt_i / sqrt d, kt_i the
    row's probability-weighted key (the oracle's attention with the keys as
    values), and the GPU's rows are held to that within the backward's bf16
    bound.  On a sharp row (one key takes almost all the weight) dP_it - D_i
    nearly cancels, so this shift is the whole gradient there: a few 1e-2
    at most, against ~4e-3 for an ordinary row of a 10 M-key head (printed).
    """
    d, Ns, Nc, rho, gamma = case
    B, H, b = 1, 1, 256
    print("largest head span backward: d %d Ns %d Nc %d" % (d, Ns, Nc), flush=True)
    dev = torch.device("cuda:0")
    Qd, Kd, Vd = make_inputs_device(B, H, d, Ns, Nc, 5252 + d, dev, "bf16")
    g = torch.Generator(device=dev).manual_seed(53 + d)
    dOd = torch.randn(Qd.shape, generator=g, device=dev).to(torch.bfloat16)
    O, ws = isa.attention(Qd, Kd, Vd, b, rho, gamma)
    dQ, dK, dV, _ = isa.backward(Qd, Kd, Vd, O, dOd, ws, b, rho, gamma)
    torch.cuda.synchronize()
    views = isa.plan_views(Qd, Kd, ws, b, rho, gamma)
    kept = views["kept_ctx"][0, 0].cpu().numpy()
    full = views["full_q"][0, 0].cpu().numpy()
    tayl = views["taylor_q"][0, 0].cpu().numpy()
    src, ctx = orc.block_ranges(Ns, Nc, b)
    # the two sums and the pruned rows, on the GPU in fp64
    dK64, dV64, dO64 = dK[0, 0].double(), dV[0, 0].double(), dOd[0, 0].double()
    vmax = float(Vd.float().abs().max())
    dv_gap = (dV64.sum(0) - dO64.sum(0)).abs()
    dv_tol = 2.0 ** -9 * (dO64.abs().sum(0) + dV64.abs().sum(0))
    dk_gap = dK64.sum(0).abs()
    dk_tol = 2.0 ** -9 * dK64.abs().sum(0) + 2.0 ** -7 * vmax * (
        dO64.abs().sum(1, keepdim=True) * Qd[0, 0].double().abs()).sum(0) / np.sqrt(d)
    print("  sum dV - sum dO: max %.3g (bound %.3g); sum dK: max %.3g (bound %.3g)" % (
        float(dv_gap.max()), float(dv_tol.min()), float(dk_gap.max()), float(dk_tol.min())), flush=True)
    assert bool((dv_gap <= dv_tol).all()) and bool((dk_gap <= dk_tol).all())
    keep = set(int(c) for c in kept)
    for c, (s, e) in enumerate(ctx):
        if c not in keep:
            assert not bool(dK[0, 0, s:e].any()) and not bool(dV[0, 0, s:e].any()), c
    del dK64, dV64, dO64
    # dQ of sampled rows against the oracle's row gradients
    rng = np.random.default_rng(6)
    full_rows = []
    for i in (int(full[0]), int(full[1]), int(full[-2]), int(full[-1])):
        s, e = src[i]
        full_rows += [s, e - 1]
    taylor_rows = np.concatenate([np.arange(s, e) for s, e in (src[int(t)] for t in tayl[:: max(1, len(tayl) // 64)])])
    tay_rows = np.array(sorted(set(rng.choice(taylor_rows, 256, replace=False).tolist())))
    full_rows = np.array(sorted(full_rows))
    Q = Qd[0, 0].double().cpu().numpy()
    K = Kd[0, 0].double().cpu().numpy()
    V = Vd[0, 0].double().cpu().numpy()
    dO = dOd[0, 0].double().cpu().numpy()
    dQh = dQ[0, 0].float().cpu().numpy()
    Oh = O[0, 0].double().cpu().numpy()
    del Qd, Kd, Vd, O, ws, dQ, dK, dV, dOd
    torch.cuda.empty_cache()
    print("  oracle row gradients", flush=True)
    kept_blocks = src + [ctx[int(c)] for c in kept]
    tok = np.concatenate([np.arange(s, e) for s, e in kept_blocks])
    Kt, Vt = K[tok], V[tok]
    qf, gf = Q[full_rows], dO[full_rows]
    dq_full, _, _ = bwd.full_attention_rows_backward(qf, Kt, Vt, gf)
    o_full, kt_full = orc.full_attention_rows(qf, Kt, Vt), orc.full_attention_rows(qf, Kt, Kt)
    del Kt, Vt
    kbar, n = orc.pool_blocks(K, kept_blocks)
    vbar, _ = orc.pool_blocks(V, kept_blocks)
    qt, gt = Q[tay_rows], dO[tay_rows]
    dq_tay, _, _ = bwd.taylor_attention_rows_backward(qt, kbar, vbar, n, gt)
    o_tay, kt_tay = orc.taylor_attention_rows(qt, kbar, vbar, n), orc.taylor_attention_rows(qt, kbar, kbar, n)
    rows = np.concatenate([full_rows, tay_rows])
    ref = np.concatenate([dq_full, dq_tay])
    dD = (np.concatenate([gf, gt]) * (Oh[rows] - np.concatenate([o_full, o_tay]))).sum(axis=1)
    shift = -dD[:, None] * np.concatenate([kt_full, kt_tay]) / np.sqrt(d)
    raw_maxrel, raw_rel = _grad_errors(dQh[rows], ref)
    maxrel, rel = _grad_errors(dQh[rows], ref + shift)
    print("  dQ rows against the exact-D oracle: max/scale %.2e rel-L2 %.2e; largest D shift %.2e (row gradients "
          "up to %.2e)" % (raw_maxrel, raw_rel, float(np.abs(shift).max()), float(np.abs(ref).max())), flush=True)
    print("  dQ rows against the oracle moved to the output's D: max/scale %.2e rel-L2 %.2e" % (maxrel, rel),
          flush=True)
    assert maxrel <= GRAD_MAXREL and rel <= GRAD_RELL2, (maxrel, rel)


def test_most_heads_fp8():
    """The FP8 variant at B*H = 65535 (its packing pass also puts B*H on grid
    y): every head's plan and Taylor rows equal isa_attention's bit for bit;
    every full-route row of the sampled heads meets test_gpu_fp8's per-row
    bound against the FP8 reference, and those rows together meet its rel-L2
    bounds (bf16's 1e-2 against the FP8 reference, 6 % against exact
    attention).  A head here has three full-route rows, too few for a rel-L2
    of its own: one allowed rounding flip moves it by several percent."""
    from oracle import isa_oracle_fp8 as f8
    from tests.parity_util import BF16_RELL2, out_errors
    from tests.test_gpu_fp8 import FP8_VS_EXACT_RELL2, _fp8_row_ratio
    B, H, d, Ns, Nc, b, rho, gamma = 1, MAX_BH, 128, 7, 5, 3, 0.5, 0.4
    print("heads limit fp8", flush=True)
    Q, K, V = make_inputs(B, H, d, Ns, Nc, seed=99, dtype="bf16")
    Qd, Kd, Vd = (device_tensor(t, "bf16") for t in (Q, K, V))
    O8, ws8, _ = isa.attention_fp8(Qd, Kd, Vd, b, rho, gamma)
    O, ws = isa.attention(Qd, Kd, Vd, b, rho, gamma)
    torch.cuda.synchronize()
    v8 = isa.plan_views(Qd, Kd, ws8, b, rho, gamma)
    v = isa.plan_views(Qd, Kd, ws, b, rho, gamma)
    for key in ("sal", "kept_ctx", "sh", "full_q", "taylor_q"):
        assert torch.equal(v8[key], v[key]), key
    full = v["full_q"][0].cpu().numpy()          # [H, kq] block indices
    kept = v["kept_ctx"][0].cpu().numpy()
    O8h, Oh = O8[0].float().cpu().numpy(), O[0].float().cpu().numpy()
    on_full = np.zeros((H, Ns), dtype=bool)
    for j in range(full.shape[1]):
        for u in range(b):
            r = full[:, j] * b + u
            ok = r < Ns
            on_full[np.nonzero(ok)[0], r[ok]] = True
    np.testing.assert_array_equal(O8h[~on_full], Oh[~on_full])
    src, ctx = orc.block_ranges(Ns, Nc, b)
    got, refs, exact, worst = [], [], [], 0.0
    for h in _sample_heads(H):
        rows = np.nonzero(on_full[h])[0]
        if rows.size == 0:
            continue
        tok = np.concatenate([np.arange(Ns)] + [np.arange(*ctx[int(c)]) for c in kept[h]])
        ref8 = f8.fp8_full_attention_rows(Q[0, h, rows], K[0, h, tok], V[0, h, tok])
        ratio, _ = _fp8_row_ratio(O8h[h, rows], ref8, Q[0, h, rows], K[0, h, tok], V[0, h, tok])
        assert ratio <= 1.0, (h, ratio)
        worst = max(worst, ratio)
        got.append(O8h[h, rows])
        refs.append(ref8)
        exact.append(orc.full_attention_rows(np.asarray(Q[0, h, rows], np.float64), K[0, h, tok], V[0, h, tok]))
    rel8 = out_errors(np.concatenate(got), np.concatenate(refs))[1]
    rel_exact = out_errors(np.concatenate(got), np.concatenate(exact))[1]
    print("  worst error / row bound %.3f, rel-L2 against the FP8 reference %.4f, against exact %.4f" % (
        worst, rel8, rel_exact), flush=True)
    assert rel8 <= BF16_RELL2 and rel_exact <= FP8_VS_EXACT_RELL2


@pytest.mark.parametrize("case", SPAN_CASES[:1], ids=lambda c: "d%d_Ns%d_Nc%d" % c[:3])
def test_largest_head_span_fp8(case):
    """The FP8 variant on the largest head span at d = 128, where its
    ping-pong kernel addresses the e4m3 key and value copies with 32-bit
    offsets (at d = 64 its kernel forms 64-bit ones): plan and Taylor rows
    equal to isa_attention's bit for bit (every row), and 8 full-route rows
    (over all 5.2 M kept tokens) within test_gpu_fp8's per-row bound of the
    FP8 reference, their rel-L2 within 1e-2 of it and 6 % of exact
    attention.  (Measured at d = 64 as well while it was written: bound
    ratio 0.06, rel-L2 1.2e-3 and 2.7 %.)"""
    from oracle import isa_oracle_fp8 as f8
    from tests.parity_util import BF16_RELL2, out_errors
    from tests.test_gpu_fp8 import FP8_VS_EXACT_RELL2, _fp8_row_ratio
    d, Ns, Nc, rho, gamma = case
    B, H, b = 1, 1, 256
    print("largest head span fp8: d %d Ns %d Nc %d" % (d, Ns, Nc), flush=True)
    dev = torch.device("cuda:0")
    Qd, Kd, Vd = make_inputs_device(B, H, d, Ns, Nc, 6262 + d, dev, "bf16")
    O8, ws8, _ = isa.attention_fp8(Qd, Kd, Vd, b, rho, gamma)
    O, ws = isa.attention(Qd, Kd, Vd, b, rho, gamma)
    torch.cuda.synchronize()
    v8 = isa.plan_views(Qd, Kd, ws8, b, rho, gamma)
    v = isa.plan_views(Qd, Kd, ws, b, rho, gamma)
    for key in ("sal", "kept_ctx", "sh", "full_q", "taylor_q"):
        assert torch.equal(v8[key], v[key]), key
    full = v["full_q"][0, 0].cpu().numpy()
    kept = v["kept_ctx"][0, 0].cpu().numpy()
    on_full = torch.zeros(Ns, dtype=torch.bool, device=dev)
    for i in full:
        on_full[int(i) * b:min((int(i) + 1) * b, Ns)] = True
    assert torch.equal(O8[0, 0][~on_full], O[0, 0][~on_full])
    src, ctx = orc.block_ranges(Ns, Nc, b)
    rows = []
    for i in (int(full[0]), int(full[1]), int(full[-2]), int(full[-1])):
        s, e = src[i]
        rows += [s, e - 1]
    rows = np.array(sorted(rows))
    O8h = O8[0, 0].float().cpu().numpy()[rows]
    Q = Qd[0, 0].double().cpu().numpy()[rows]
    tok = torch.from_numpy(np.concatenate([np.arange(Ns)] + [np.arange(*ctx[int(c)]) for c in kept])).to(dev)
    Kt = Kd[0, 0][tok].double().cpu().numpy()
    Vt = Vd[0, 0][tok].double().cpu().numpy()
    del Qd, Kd, Vd, O8, O, ws8, ws, tok
    torch.cuda.empty_cache()
    print("  fp8 reference rows", flush=True)
    ref8 = f8.fp8_full_attention_rows(Q, Kt, Vt)
    ratio, _ = _fp8_row_ratio(O8h, ref8, Q, Kt, Vt)
    rel8 = out_errors(O8h, ref8)[1]
    rel_exact = out_errors(O8h, orc.full_attention_rows(Q, Kt, Vt))[1]
    print("  worst error / row bound %.3f, rel-L2 against the FP8 reference %.4f, against exact %.4f" % (
        ratio, rel8, rel_exact), flush=True)
    assert ratio <= 1.0 and rel8 <= BF16_RELL2 and rel_exact <= FP8_VS_EXACT_RELL2
