"""GPU parity of the backward pass (through the C-ABI) against the fp64 oracle.

The oracle differentiates the forward definitions with the plan frozen
(oracle/isa_oracle_backward.py); it is run with the GPU's own kept_ctx and
full_q, so a tie that flips under rounding cannot fail the float check (the
forward tests check the sets themselves).

Tolerance, per gradient tensor: the kernels round p and ds to bf16 before
their MFMA contractions (2^-9 relative each), accumulate in fp32 and round
the result to bf16 (2^-9), with bf16 inputs on both sides.  Each term thus
carries about 4e-3 relative error, sums of many terms of mixed sign keep
that order relative to the tensor's scale, so the bound is
    ||g - g_ref||_2 <= 1.5e-2 ||g_ref||_2   and   max|g - g_ref| <= 3e-2 max|g_ref|.
"""

import numpy as np
import pytest
import torch

from oracle import isa_oracle as orc
from oracle import isa_oracle_backward as bwd
from sparse_attention_context_amd import isa
from sparse_attention_context_amd.synth import make_inputs, round_to_bf16
from tests.parity_util import device_tensor

pytestmark = pytest.mark.gpu

GRAD_RELL2 = 1.5e-2
GRAD_MAXREL = 3e-2


def _report(msg):
    print(msg, flush=True)


def _grad_errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = max(float(np.max(np.abs(ref))), 1e-30)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    return float(np.max(np.abs(got - ref))) / scale, rel


def _assert_grad(name, got, ref):
    maxrel, rel = _grad_errors(got, ref)
    assert maxrel <= GRAD_MAXREL and rel <= GRAD_RELL2, (name, maxrel, rel)
    return maxrel, rel


def _run(B, H, d, Ns, Nc, b, rho, gamma, seed, two_call=False):
    Q, K, V = make_inputs(B, H, d, Ns, Nc, seed=seed, dtype="bf16")
    dO = round_to_bf16(np.random.default_rng(seed + 1).standard_normal((B, H, Ns, d)))
    Qd, Kd, Vd, dOd = (device_tensor(t, "bf16") for t in (Q, K, V, dO))
    if two_call:
        ws = isa.plan(Qd, Kd, Vd, b, rho, gamma)
        O = isa.forward(Qd, Kd, Vd, ws, b, rho, gamma)
    else:
        O, ws = isa.attention(Qd, Kd, Vd, b, rho, gamma)
    dQ, dK, dV, bws = isa.backward(Qd, Kd, Vd, O, dOd, ws, b, rho, gamma)
    torch.cuda.synchronize()
    return (Q, K, V, dO), (Qd, Kd, Vd, dOd, O, ws, bws), (dQ, dK, dV)


CASES = [
    # B, H, d, Ns, Nc, b, rho, gamma
    (1, 2, 64, 256, 256, 16, 0.5, 0.25),
    (2, 3, 128, 1000, 700, 64, 0.25, 0.2),
    (1, 2, 128, 777, 333, 128, 0.3, 0.5),       # ragged tails, b above the key tile
    (1, 2, 64, 150, 100, 1, 0.4, 0.3),          # b = 1
    (1, 2, 64, 500, 0, 32, 0.5, 0.3),           # no context
    (1, 2, 128, 640, 640, 64, 0.0, 0.0),        # no context kept, all Taylor
    (1, 2, 128, 640, 577, 64, 1.0, 1.0),        # dense limit: no Taylor rows
    (1, 2, 128, 1000, 900, 200, 0.5, 0.5),      # short kept tail block inside a key tile
    (1, 1, 128, 3000, 2500, 64, 0.25, 0.2),     # several dQ splits and dK/dV key tiles
    (1, 2, 128, 150, 100, 1, 0.4, 0.3),         # b = 1 at d = 128: route rows one by one
    (1, 2, 128, 500, 0, 32, 0.5, 0.3),          # no context at d = 128
    (1, 2, 128, 700, 630, 50, 1.0, 0.5),        # short last context block kept; row tiles straddle blocks
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dd%d_Ns%d_Nc%d_b%d_r%g_g%g" % c)
def test_backward_elementwise(case):
    B, H, d, Ns, Nc, b, rho, gamma = case
    _report("backward case %s" % (case,))
    (Q, K, V, dO), (Qd, Kd, Vd, dOd, O, ws, bws), (dQ, dK, dV) = _run(*case, seed=Ns + 3 * Nc + d)
    views = isa.plan_views(Qd, Kd, ws, b, rho, gamma)
    kept = views["kept_ctx"].cpu().numpy()
    full = views["full_q"].cpu().numpy()
    rQ, rK, rV = bwd.oracle_backward(Q, K, V, dO, b, kept, full)
    for name, g, r in (("dQ", dQ, rQ), ("dK", dK, rK), ("dV", dV, rV)):
        maxrel, rel = _assert_grad(name, g.float().cpu().numpy(), r)
        _report("  %s max/scale %.2e rel-L2 %.2e" % (name, maxrel, rel))
    # rows of pruned context blocks are exactly zero
    src, ctx = orc.block_ranges(Ns, Nc, b)
    dKh, dVh = dK.float().cpu().numpy(), dV.float().cpu().numpy()
    for x in range(B):
        for h in range(H):
            keep = set(int(c) for c in kept[x, h])
            for c, (s, e) in enumerate(ctx):
                if c not in keep:
                    assert not dKh[x, h, s:e].any() and not dVh[x, h, s:e].any()


def test_backward_two_call_workspace_and_repeat_are_bitwise_equal():
    case = (1, 2, 128, 1000, 700, 64, 0.25, 0.2)
    _, (Qd, Kd, Vd, dOd, O, ws, bws), grads = _run(*case, seed=5)
    _, (_, _, _, _, O2, ws2, _), grads2 = _run(*case, seed=5, two_call=True)
    assert torch.equal(O, O2)
    for g, g2 in zip(grads, grads2):
        assert torch.equal(g, g2)
    b, rho, gamma = case[5:]
    again = isa.backward(Qd, Kd, Vd, O, dOd, ws, b, rho, gamma, bwd_workspace=bws)
    torch.cuda.synchronize()
    for g, g2 in zip(grads, again[:3]):
        assert torch.equal(g, g2)


def test_backward_stage_sequence_equals_backward():
    case = (1, 2, 128, 1000, 700, 64, 0.25, 0.2)
    _, (Qd, Kd, Vd, dOd, O, ws, bws), grads = _run(*case, seed=9)
    b, rho, gamma = case[5:]
    dQ, dK, dV = torch.empty_like(Qd), torch.empty_like(Kd), torch.empty_like(Vd)
    for name in isa.BWD_STAGES:
        isa.run_backward_stage(name, Qd, Kd, Vd, O, dOd, ws, bws, dQ, dK, dV, b, rho, gamma)
    torch.cuda.synchronize()
    for g, g2 in zip(grads, (dQ, dK, dV)):
        assert torch.equal(g, g2)


def test_backward_video_dit_layer_full_heads():
    """The benchmarked video-DiT layer (B1 H24 d128, 17550 + 17550 rows, b64,
    rho .25, gamma .2): every head checked by properties that hold at any size
    (the keys' gradients sum to zero, the values' to the sum of dO), and two
    whole heads element by element against the oracle."""
    from sparse_attention_context_amd.configs import BY_NAME
    from sparse_attention_context_amd.synth import workload_inputs
    w = BY_NAME["video_dit_layer"]
    _report("backward video-DiT layer: inputs")
    Q, K, V = workload_inputs(w)
    dO = round_to_bf16(np.random.default_rng(123).standard_normal(Q.shape))
    Qd, Kd, Vd, dOd = (device_tensor(t, "bf16") for t in (Q, K, V, dO))
    O, ws = isa.attention(Qd, Kd, Vd, w.b, w.rho, w.gamma)
    dQ, dK, dV, _ = isa.backward(Qd, Kd, Vd, O, dOd, ws, w.b, w.rho, w.gamma)
    torch.cuda.synchronize()
    _report("backward video-DiT layer: GPU done")
    views = isa.plan_views(Qd, Kd, ws, w.b, w.rho, w.gamma)
    dKs = dK.float().sum(dim=2)
    dVs = dV.float().sum(dim=2)
    dOs = torch.from_numpy(dO).to(dK.device).float().sum(dim=2)
    kn = dK.float().norm(dim=(2, 3))
    assert float(((dKs.norm(dim=2)) / kn).max()) <= 5e-2
    assert float(((dVs - dOs).norm(dim=2) / dOs.norm(dim=2)).max()) <= 2e-2
    kept = views["kept_ctx"].cpu().numpy()
    full = views["full_q"].cpu().numpy()
    for h in (0, w.H - 1):
        rQ, rK, rV = bwd.oracle_backward_head(Q[0, h], K[0, h], V[0, h], dO[0, h], w.b, kept[0, h], full[0, h])
        for name, g, r in (("dQ", dQ, rQ), ("dK", dK, rK), ("dV", dV, rV)):
            maxrel, rel = _assert_grad(name, g[0, h].float().cpu().numpy(), r)
            _report("  head %d %s max/scale %.2e rel-L2 %.2e" % (h, name, maxrel, rel))
