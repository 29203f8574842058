"""GPU parity of the FP8 variant of the full route (isa_attention_fp8).

The plan and the Taylor rows are those of isa_attention, bit for bit.  The
full-route rows are compared with the FP8 reference (oracle/isa_oracle_fp8.py:
the same e4m3 rounding and block scales, fp64 otherwise).  The two differ in
the fp32 accumulation of the logits and in exp2's last bit, so a probability
that sits on an e4m3 rounding midpoint can round one step (2^-4 of itself)
the other way on one side: that moves one output element by at most
2^-4 max|V|.  Bound: rel-L2 <= 1e-2 (as bf16) and max-abs <= 2^-4 max|V| +
2e-2.  The error against exact attention is the variant's own (a few percent
of the output norm) and is bounded separately."""

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


def _assert_fp8(got, ref, Vt):
    maxabs, rel = out_errors(got, ref)
    bound = 2.0 ** -4 * float(np.abs(Vt).max()) + BF16_MAXABS
    assert maxabs <= bound and rel <= BF16_RELL2, (maxabs, bound, rel)
    return maxabs, rel


def _full_rows(full_q, b, Ns):
    return np.array([r for i in full_q for r in range(int(i) * b, min((int(i) + 1) * b, Ns))], dtype=np.int64)


@pytest.mark.parametrize("case", [
    (1, 2, 128, 1000, 700, 64, 0.25, 0.2),
    (2, 3, 64, 777, 333, 48, 0.3, 0.5),
    (1, 2, 128, 1000, 900, 200, 0.5, 0.5),       # short kept tail block
    (1, 2, 128, 640, 577, 64, 1.0, 1.0),         # every block on the full route
    (1, 1, 128, 3000, 2500, 64, 0.25, 0.2),      # split key range
], ids=lambda c: "B%dH%dd%d_Ns%d_Nc%d_b%d_r%g_g%g" % c)
def test_fp8_full_route(case):
    B, H, d, Ns, Nc, b, rho, gamma = case
    print("fp8 case %s" % (case,), flush=True)
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
            maxabs, rel = _assert_fp8(O8h[x, h, rows], ref8, V[x, h, tok])
            exact = orc.full_attention_rows(np.asarray(Q[x, h, rows], np.float64), K[x, h, tok], V[x, h, tok])
            _, rel_exact = out_errors(O8h[x, h, rows], exact)
            print("  head %d,%d: vs fp8 reference max %.2e rel %.2e; vs exact rel %.3f" % (x, h, maxabs, rel, rel_exact),
                  flush=True)
            assert rel_exact <= FP8_VS_EXACT_RELL2


def test_fp8_video_dit_layer_sampled_rows():
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
    for h in (0, 11, 23):
        full = v["full_q"][0, h].cpu().numpy()
        kept = v["kept_ctx"][0, h].cpu().numpy()
        rows = rng.choice(_full_rows(full, w.b, w.Ns), 64, replace=False)
        src, ctx = orc.block_ranges(w.Ns, w.Nc, w.b)
        tok = np.concatenate([np.arange(w.Ns)] + [np.arange(*ctx[int(c)]) for c in kept])
        ref8 = f8.fp8_full_attention_rows(Q[0, h, rows], K[0, h, tok], V[0, h, tok])
        _assert_fp8(O8h[0, h, rows], ref8, V[0, h, tok])
        exact = orc.full_attention_rows(np.asarray(Q[0, h, rows], np.float64), K[0, h, tok], V[0, h, tok])
        assert out_errors(O8h[0, h, rows], exact)[1] <= FP8_VS_EXACT_RELL2
