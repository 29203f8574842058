"""isa_attention_noalloc against isa_attention, through the C-ABI.

The entry point for callers that cannot allocate runs the layer's kernels in
the library's fixed scratch array; its output must equal isa_attention's bit
for bit (same kernels, same arithmetic).  Three calls in a row, each on a
smaller layer than the one before, so that a call that depended on what the
previous one left in the scratch would differ."""

import pytest
import torch

from sparse_attention_context_amd import isa
from sparse_attention_context_amd.synth import make_inputs
from tests.parity_util import device_tensor

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, d, Ns, Nc, b, rho, gamma, dtype
    (1, 8, 128, 4000, 3000, 64, 0.25, 0.2, "bf16"),
    (1, 2, 128, 1000, 700, 64, 0.5, 0.4, "bf16"),
    (1, 2, 64, 300, 200, 16, 0.5, 0.25, "f32"),
]


def test_noalloc_matches_attention_on_successive_calls():
    outs = []
    for case in CASES:
        B, H, d, Ns, Nc, b, rho, gamma, dtype = case
        print("noalloc case %s" % (case,), flush=True)
        Q, K, V = (device_tensor(t, dtype) for t in make_inputs(B, H, d, Ns, Nc, seed=Ns + 7, dtype=dtype))
        desc = isa.desc_for(Q, K, b, rho, gamma, V=V)
        assert isa.workspace_size(desc) <= isa.noalloc_scratch_bytes()
        O = torch.full_like(Q, float("nan"))
        isa.attention_noalloc(Q, K, V, b, rho, gamma, out=O)
        O_ref, _ = isa.attention(Q, K, V, b, rho, gamma)
        torch.cuda.synchronize()
        assert torch.equal(O, O_ref), case
        outs.append((Q, K, V, O_ref, case))
    # and again in reverse size order: the first layer after the smallest
    Q, K, V, O_ref, case = outs[0]
    O = torch.empty_like(Q)
    isa.attention_noalloc(Q, K, V, case[5], case[6], case[7], out=O)
    torch.cuda.synchronize()
    assert torch.equal(O, O_ref)


def test_noalloc_strided_views():
    """The same entry point on [B,N,H,d] views (tokens before heads)."""
    B, H, d, Ns, Nc, b, rho, gamma = 1, 3, 128, 1000, 700, 64, 0.25, 0.2
    Q, K, V = (device_tensor(t, "bf16") for t in make_inputs(B, H, d, Ns, Nc, seed=5, dtype="bf16"))
    O_ref, _ = isa.attention(Q, K, V, b, rho, gamma)
    tm = [t.transpose(1, 2).contiguous().transpose(1, 2) for t in (Q, K, V)]
    O = torch.empty_like(Q).transpose(1, 2).contiguous().transpose(1, 2)
    isa.attention_noalloc(*tm, b, rho, gamma, out=O)
    torch.cuda.synchronize()
    assert torch.equal(O, O_ref)
