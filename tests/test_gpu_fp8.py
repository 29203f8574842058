"""GPU parity of the FP8 variant of the full route (isa_attention_fp8).

The plan and the Taylor rows are those of isa_attention, bit for bit.  The
full-route rows are compared with the FP8 reference (oracle/isa_oracle_fp8.py:
e4m3 rounding under MX block scales, fp64 otherwise) and, independently, with
exact attention.

Against the FP8 reference, per row.  The kernel's logits are fp32 sums and
its exp2 has its own last bit, so a probability p_t near an e4m3 rounding
midpoint can round one step the other way.  One step is at most p_t / 8
(three mantissa bits), so such a flip moves the row's output by at most
pi_t |v_t| / 8, pi_t = p_t / sum p the softmax probability.  The bound of a
row is therefore two such flips of its largest probability (pi_max, from
exact attention), plus bf16 output rounding:
    |o - o_ref| <= 2 * pi_max * max|V| / 8 + 2^-8 |o_ref| + 2e-3.
On a row without a sharp key, pi_max is ~1e-3 and the bound is ~2e-3.  The
rows' rel-L2 must stay within bf16's 1e-2.  Against exact attention the
variant's own rounding error (a few percent of the output norm) is bounded
at 6 %."""

import numpy as np
import pytest
import torch

from oracle import isa_oracle as orc
from oracle import isa_oracle_fp8 as f8
from sparse_attention_context_amd import isa
from sparse_attention_context_amd.synth import make_inputs
from tests.parity_util import BF16_MAXABS, BF16_RELL2, device_tensor, out_errors

pytestmark = pytest.mark.gpu

FP8_VS_EXACT_RELL2 = 6e-2


def _pi_max(q, Kt):
    """Largest softmax probability of each row (exact, fp64)."""
    x = np.asarray(q, np.float64) @ np.asarray(Kt, np.float64).T / np.sqrt(q.shape[1])
    x -= x.max(axis=1, keepdims=True)
    p = np.exp(x)
    return p.max(axis=1) / p.sum(axis=1)


def _fp8_row_ratio(got, ref, q, Kt, Vt):
    """Worst ratio of an entry's error to the per-row bound of the module
    docstring, and the largest bound."""
    got = np.asarray(got, np.float64)
    bound = (2.0 * _pi_max(q, Kt) * float(np.abs(Vt).max()) / 8.0)[:, None] + 2.0 ** -8 * np.abs(ref) + 2e-3
    return float((np.abs(got - ref) / bound).max()), float(bound.max())


def _assert_fp8(got, ref, q, Kt, Vt):
    """Per-row bound of the module docstring and the rows' rel-L2; returns
    (maxabs, rel, worst ratio of a row's error to its bound, largest bound)."""
    ratio, bmax = _fp8_row_ratio(got, ref, q, Kt, Vt)
    maxabs, rel = out_errors(got, ref)
    assert ratio <= 1.0 and rel <= BF16_RELL2, (maxabs, ratio, rel)
    return maxabs, rel, ratio, bmax


def _full_rows(full_q, b, Ns):
    return np.array([r for i in full_q for r in range(int(i) * b, min((int(i) + 1) * b, Ns))], dtype=np.int64)


@pytest.mark.parametrize("case", [
    (1, 2, 128, 1000, 700, 64, 0.25, 0.2),
    (2, 3, 64, 777, 333, 48, 0.3, 0.5),
    (1, 2, 128, 1000, 900, 200, 0.5, 0.5),       # short kept tail block
    (1, 2, 128, 640, 577, 64, 1.0, 1.0),         # every block on the full route
    (1, 1, 128, 3000, 2500, 64, 0.25, 0.2),      # split key range
], ids=lambda c: "B%dH%dd%d_Ns%d_Nc%d_b%d_r%g_g%g" % c)
def test_fp8_full_route(case, parity_record):
    B, H, d, Ns, Nc, b, rho, gamma = case
    print("fp8 case %s" % (case,), flush=True)
    rec = {"case": "fp8 B%dH%dd%d_Ns%d_Nc%d_b%d_r%g_g%g" % case, "rel_l2_vs_exact": 0.0, "maxabs_vs_fp8_ref": 0.0,
           "rel_l2_vs_fp8_ref": 0.0, "largest_row_bound": 0.0}
    worst = 0.0
    Q, K, V = make_inputs(B, H, d, Ns, Nc, seed=Ns + Nc + 1, dtype="bf16")
    Qd, Kd, Vd = (device_tensor(t, "bf16") for t in (Q, K, V))
    O8, ws8, _ = isa.attention_fp8(Qd, Kd, Vd, b, rho, gamma)
    O, ws = isa.attention(Qd, Kd, Vd, b, rho, gamma)
    torch.cuda.synchronize()
    v8 = isa.plan_views(Qd, Kd, ws8, b, rho, gamma)
    v = isa.plan_views(Qd, Kd, ws, b, rho, gamma)
    for key in ("sal", "kept_ctx", "sh", "full_q", "taylor_q"):
        assert torch.equal(v8[key], v[key]), key
    O8h, Oh = O8.float().cpu().numpy(), O.float().cpu().numpy()
    for x in range(B):
        for h in range(H):
            full = v["full_q"][x, h].cpu().numpy()
            kept = v["kept_ctx"][x, h].cpu().numpy()
            rows = _full_rows(full, b, Ns)
            tay = np.setdiff1d(np.arange(Ns), rows)
            np.testing.assert_array_equal(O8h[x, h, tay], Oh[x, h, tay])
            if rows.size == 0:
                continue
            src, ctx = orc.block_ranges(Ns, Nc, b)
            tok = np.concatenate([np.arange(Ns)] + [np.arange(*ctx[int(c)]) for c in kept])
            ref8 = f8.fp8_full_attention_rows(Q[x, h, rows], K[x, h, tok], V[x, h, tok])
            maxabs, rel, ratio, bmax = _assert_fp8(O8h[x, h, rows], ref8, Q[x, h, rows], K[x, h, tok], V[x, h, tok])
            exact = orc.full_attention_rows(np.asarray(Q[x, h, rows], np.float64), K[x, h, tok], V[x, h, tok])
            _, rel_exact = out_errors(O8h[x, h, rows], exact)
            worst = max(worst, ratio)
            rec["rel_l2_vs_exact"] = max(rec["rel_l2_vs_exact"], rel_exact)
            rec["maxabs_vs_fp8_ref"] = max(rec["maxabs_vs_fp8_ref"], maxabs)
            rec["rel_l2_vs_fp8_ref"] = max(rec["rel_l2_vs_fp8_ref"], rel)
            rec["largest_row_bound"] = max(rec["largest_row_bound"], bmax)
            assert rel_exact <= FP8_VS_EXACT_RELL2
    rec["worst_error_over_row_bound"] = worst
    parity_record(rec)


def test_fp8_video_dit_layer_sampled_rows(parity_record):
    from sparse_attention_context_amd.configs import BY_NAME
    from sparse_attention_context_amd.synth import workload_inputs
    w = BY_NAME["video_dit_layer"]
    Q, K, V = workload_inputs(w)
    Qd, Kd, Vd = (device_tensor(t, "bf16") for t in (Q, K, V))
    O8, ws8, _ = isa.attention_fp8(Qd, Kd, Vd, w.b, w.rho, w.gamma)
    torch.cuda.synchronize()
    v = isa.plan_views(Qd, Kd, ws8, w.b, w.rho, w.gamma)
    rng = np.random.default_rng(0)
    O8h = O8.float().cpu().numpy()
    rec = {"case": "fp8 video_dit_layer, 64 full-route rows of heads 0, 11, 23", "worst_error_over_row_bound": 0.0,
           "rel_l2_vs_exact": 0.0}
    for h in (0, 11, 23):
        full = v["full_q"][0, h].cpu().numpy()
        kept = v["kept_ctx"][0, h].cpu().numpy()
        rows = rng.choice(_full_rows(full, w.b, w.Ns), 64, replace=False)
        src, ctx = orc.block_ranges(w.Ns, w.Nc, w.b)
        tok = np.concatenate([np.arange(w.Ns)] + [np.arange(*ctx[int(c)]) for c in kept])
        ref8 = f8.fp8_full_attention_rows(Q[0, h, rows], K[0, h, tok], V[0, h, tok])
        _, _, ratio, _ = _assert_fp8(O8h[0, h, rows], ref8, Q[0, h, rows], K[0, h, tok], V[0, h, tok])
        exact = orc.full_attention_rows(np.asarray(Q[0, h, rows], np.float64), K[0, h, tok], V[0, h, tok])
        rel_exact = out_errors(O8h[0, h, rows], exact)[1]
        rec["worst_error_over_row_bound"] = max(rec["worst_error_over_row_bound"], ratio)
        rec["rel_l2_vs_exact"] = max(rec["rel_l2_vs_exact"], rel_exact)
        assert rel_exact <= FP8_VS_EXACT_RELL2
    parity_record(rec)
