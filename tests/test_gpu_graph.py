"""A whole isa_attention call captured in a HIP graph and replayed.

Replays run with eager library calls, input updates and synchronisations in
between; every replay must equal the eager call on the same inputs bit for
bit (the graph holds the same kernels on the same pointers)."""

import pytest
import torch

from sparse_attention_context_amd import isa
from sparse_attention_context_amd.synth import make_inputs
from tests.parity_util import device_tensor

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case", [(1, 4, 128, 2000, 1500, 64, 0.25, 0.2, "bf16"),
                                  (1, 3, 64, 1111, 999, 48, 0.2, 0.7, "bf16"),
                                  (1, 2, 64, 300, 200, 16, 0.5, 0.25, "f32")],
                         ids=lambda c: "B%dH%dd%d_Ns%d_Nc%d_b%d_r%g_g%g_%s" % c)
def test_captured_layer_replays_match_eager(case):
    B, H, d, Ns, Nc, b, rho, gamma, dtype = case
    print("graph case %s" % (case,), flush=True)
    inputs = [tuple(device_tensor(t, dtype) for t in make_inputs(B, H, d, Ns, Nc, seed=s, dtype=dtype))
              for s in (1, 2, 3)]
    Q, K, V = (t.clone() for t in inputs[0])
    layer = isa.CapturedAttention(Q, K, V, b, rho, gamma)
    for rep in range(4):
        Qi, Ki, Vi = inputs[rep % 3]
        Q.copy_(Qi)
        K.copy_(Ki)
        V.copy_(Vi)
        O = layer.replay().clone()
        # eager work between the replays
        O_ref, ws_ref = isa.attention(Qi, Ki, Vi, b, rho, gamma)
        torch.cuda.synchronize()
        assert torch.equal(O, O_ref), rep
        v1 = isa.plan_views(Q, K, layer.workspace, b, rho, gamma)
        v2 = isa.plan_views(Qi, Ki, ws_ref, b, rho, gamma)
        for key in ("kept_ctx", "full_q", "sh", "sal"):
            assert torch.equal(v1[key], v2[key]), (rep, key)
