"""GPU parity of the context-token query rows (isa_context_forward) against
the oracle (reading N2: ordinary attention of each context row over all
keys), element by element on small shapes and on sampled rows of the
benchmarked video-DiT layer.  Tolerances are the forward's (bf16)."""

import numpy as np
import pytest
import torch

from oracle import isa_oracle as orc
from sparse_attention_context_amd import isa
from sparse_attention_context_amd.synth import make_inputs
from tests.parity_util import assert_output, device_tensor

pytestmark = pytest.mark.gpu


def _context_queries(B, H, d, Nc, seed):
    return np.ascontiguousarray(make_inputs(B, H, d, Nc, 0, seed=seed, dtype="bf16")[0])


@pytest.mark.parametrize("case", [
    (1, 2, 64, 300, 200), (2, 3, 128, 1000, 700), (1, 2, 128, 77, 1333), (1, 1, 64, 1, 1), (1, 2, 128, 640, 577),
], ids=lambda c: "B%dH%dd%d_Ns%d_Nc%d" % c)
def test_context_rows_elementwise(case):
    B, H, d, Ns, Nc = case
    print("context case %s" % (case,), flush=True)
    _, K, V = make_inputs(B, H, d, Ns, Nc, seed=Ns + Nc, dtype="bf16")
    Qc = _context_queries(B, H, d, Nc, seed=Nc + 1)
    Qd, Kd, Vd = (device_tensor(t, "bf16") for t in (Qc, K, V))
    Oc = isa.context_forward(Qd, Kd, Vd)
    torch.cuda.synchronize()
    got = Oc.float().cpu().numpy()
    for x in range(B):
        for h in range(H):
            assert_output(got[x, h], orc.context_rows_forward(Qc[x, h], K[x, h], V[x, h]), "bf16")


def test_context_rows_video_dit_layer_sampled():
    from sparse_attention_context_amd.configs import BY_NAME
    from sparse_attention_context_amd.synth import workload_inputs
    w = BY_NAME["video_dit_layer"]
    _, K, V = workload_inputs(w)
    Qc = _context_queries(w.B, w.H, w.d, w.Nc, seed=99)
    Qd, Kd, Vd = (device_tensor(t, "bf16") for t in (Qc, K, V))
    Oc = isa.context_forward(Qd, Kd, Vd)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.concatenate([rng.choice(w.Nc, 48, replace=False), [0, w.Nc - 1]])
    got = Oc.float().cpu().numpy()
    for h in range(w.H):
        assert_output(got[0, h, rows], orc.context_rows_forward(Qc[0, h, rows], K[0, h], V[0, h]), "bf16")
