"""GPU parity of strided tensors through the C-ABI (isa_desc.q/.k/.v/.o).

An attention layer usually holds Q, K and V as [B,N,H,d] (tokens before
heads, as a fused projection writes them), and the in-context layer
concatenates source and context tokens ("Lightning Unified Video Editing via
In-Context Sparse Attention", English abstract).  The library reads such
views in place: each case runs the layer on views -- X.transpose(1, 2) of a
[B,N,H,d] tensor, slices of one fused [B,N,3,H,d] buffer, rows padded in
memory -- and requires the output, the plan and the gradients to equal
those of the contiguous call bit for bit (the kernels' arithmetic does not
depend on the addressing), and the output to match the oracle.
"""

import numpy as np
import pytest
import torch

from oracle import isa_oracle as orc
from sparse_attention_context_amd import isa
from sparse_attention_context_amd.synth import make_inputs
from tests.parity_util import assert_output, device_tensor

pytestmark = pytest.mark.gpu

PLAN_KEYS = ("sal", "kept_ctx", "sh", "full_q", "taylor_q")


def _token_major(x):
    """[B,H,N,d] -> the same values as a transposed view of a [B,N,H,d] tensor."""
    return x.transpose(1, 2).contiguous().transpose(1, 2)


def _padded_rows(x, pad=64):
    """The same values as a view whose rows are d + pad elements apart."""
    B, H, N, d = x.shape
    buf = torch.zeros((B, H, N, d + pad), dtype=x.dtype, device=x.device)
    buf[..., :d] = x
    return buf[..., :d]


def _fused_qkv(Q, K, V):
    """Q, K, V as slices of one [B,N,3,H,d] buffer (N = K's rows; Q's rows are
    the first Ns of slot 0)."""
    B, H, Nk, d = K.shape
    Ns = Q.shape[2]
    buf = torch.zeros((B, Nk, 3, H, d), dtype=K.dtype, device=K.device)
    buf[:, :Ns, 0] = Q.transpose(1, 2)
    buf[:, :, 1] = K.transpose(1, 2)
    buf[:, :, 2] = V.transpose(1, 2)
    return buf[:, :Ns, 0].transpose(1, 2), buf[:, :, 1].transpose(1, 2), buf[:, :, 2].transpose(1, 2)


CASES = [
    # B, H, d, Ns, Nc, b, rho, gamma, dtype
    (2, 3, 128, 1000, 700, 64, 0.25, 0.2, "bf16"),
    (1, 40, 128, 2000, 1100, 64, 0.5, 1.0, "bf16"),   # the persistent full-route kernel (whole row tiles, then ranges)
    (1, 22, 128, 1000, 1100, 64, 0.5, 1.0, "bf16"),   # ranges cut row tiles into parts of 1 to 9 key tiles
    (1, 3, 64, 1111, 999, 48, 0.2, 0.7, "bf16"),
    (1, 2, 128, 333, 271, 32, 0.5, 0.4, "f32"),
    (1, 2, 64, 300, 200, 16, 0.5, 0.25, "f32"),
]
LAYOUTS = ["token_major", "padded_rows", "fused_qkv", "mixed"]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dd%d_Ns%d_Nc%d_b%d_r%g_g%g_%s" % c)
def test_strided_views_match_contiguous(case, layout):
    B, H, d, Ns, Nc, b, rho, gamma, dtype = case
    print("strided case %s %s" % (case, layout), flush=True)
    Qn, Kn, Vn = make_inputs(B, H, d, Ns, Nc, seed=Ns + Nc + 3, dtype=dtype)
    Q, K, V = (device_tensor(t, dtype) for t in (Qn, Kn, Vn))
    O, ws = isa.attention(Q, K, V, b, rho, gamma)
    if layout == "token_major":
        Qs, Ks, Vs = _token_major(Q), _token_major(K), _token_major(V)
        Os = _token_major(torch.zeros_like(Q))
    elif layout == "padded_rows":
        Qs, Ks, Vs = _padded_rows(Q), _padded_rows(K, 128), _padded_rows(V, 32)
        Os = _padded_rows(torch.zeros_like(Q), 96)
    elif layout == "fused_qkv":
        Qs, Ks, Vs = _fused_qkv(Q, K, V)
        Os = _token_major(torch.zeros_like(Q))
    else:   # K and V laid out differently (the per-item full-route kernel)
        Qs, Ks, Vs = _padded_rows(Q), _token_major(K), _padded_rows(V)
        Os = torch.zeros_like(Q)
    assert not Ks.is_contiguous()
    O2, ws2 = isa.attention(Qs, Ks, Vs, b, rho, gamma, out=Os)
    torch.cuda.synchronize()
    assert O2.data_ptr() == Os.data_ptr()
    assert torch.equal(O2, O), "strided output differs from the contiguous call"
    v1 = isa.plan_views(Q, K, ws, b, rho, gamma)
    v2 = isa.plan_views(Q, K, ws2, b, rho, gamma)
    for key in PLAN_KEYS:
        assert torch.equal(v1[key], v2[key]), key
    # the two-call path on the views
    ws3 = isa.plan(Qs, Ks, Vs, b, rho, gamma)
    O3 = isa.forward(Qs, Ks, Vs, ws3, b, rho, gamma, out=_token_major(torch.zeros_like(Q)))
    torch.cuda.synchronize()
    assert torch.equal(O3, O)
    # and the oracle, on the first head
    kept = v2["kept_ctx"][0, 0].cpu().numpy()
    full = v2["full_q"][0, 0].cpu().numpy()
    ref = orc.oracle_forward_head(Qn[0, 0], Kn[0, 0], Vn[0, 0], b, kept, full)
    assert_output(O2[0, 0].float().cpu().numpy(), ref, dtype)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_strided_dense_and_context_rows(dtype, d):
    B, H, Ns, Nc = 1, 2, 700, 450
    Qn, Kn, Vn = make_inputs(B, H, d, Ns, Nc, seed=5, dtype=dtype)
    Q, K, V = (device_tensor(t, dtype) for t in (Qn, Kn, Vn))
    O = isa.dense_forward(Q, K, V)
    O2 = isa.dense_forward(_token_major(Q), _padded_rows(K), _token_major(V), out=_padded_rows(torch.zeros_like(Q)))
    torch.cuda.synchronize()
    assert torch.equal(O, O2)
    if dtype == "bf16":
        g = torch.Generator(device="cuda").manual_seed(3)
        Qc = torch.randn((B, H, Nc, d), generator=g, device="cuda").to(torch.bfloat16)
        Oc = isa.context_forward(Qc, K, V)
        Oc2 = isa.context_forward(_token_major(Qc), _token_major(K), _padded_rows(V),
                                  out=_token_major(torch.zeros_like(Qc)))
        torch.cuda.synchronize()
        assert torch.equal(Oc, Oc2)


@pytest.mark.parametrize("case", [(1, 3, 128, 1000, 700, 64, 0.25, 0.3), (1, 2, 64, 777, 333, 48, 0.3, 0.5),
                                  (1, 8, 128, 1500, 1024, 32, 1.0, 1.0)],
                         ids=lambda c: "B%dH%dd%d_Ns%d_Nc%d_b%d_r%g_g%g" % c)
def test_strided_backward_matches_contiguous(case):
    B, H, d, Ns, Nc, b, rho, gamma = case
    print("strided backward case %s" % (case,), flush=True)
    Qn, Kn, Vn = make_inputs(B, H, d, Ns, Nc, seed=11, dtype="bf16")
    Q, K, V = (device_tensor(t, "bf16") for t in (Qn, Kn, Vn))
    g = torch.Generator(device="cuda").manual_seed(5)
    dO = torch.randn(Q.shape, generator=g, device="cuda").to(torch.bfloat16)
    O, ws = isa.attention(Q, K, V, b, rho, gamma)
    dQ, dK, dV, _ = isa.backward(Q, K, V, O, dO, ws, b, rho, gamma)
    Qs, Ks, Vs = _token_major(Q), _padded_rows(K), _token_major(V)
    Os = _token_major(torch.zeros_like(Q))
    Os, ws2 = isa.attention(Qs, Ks, Vs, b, rho, gamma, out=Os)
    dOs = torch.empty_strided(Os.shape, Os.stride(), dtype=dO.dtype, device=dO.device)
    dOs.copy_(dO)
    dQ2, dK2, dV2, _ = isa.backward(Qs, Ks, Vs, Os, dOs, ws2, b, rho, gamma)
    torch.cuda.synchronize()
    assert dQ2.stride() == Qs.stride() and dK2.stride() == Ks.stride()
    assert torch.equal(dQ, dQ2) and torch.equal(dK, dK2) and torch.equal(dV, dV2)


def test_strided_fp8_matches_contiguous():
    B, H, d, Ns, Nc, b, rho, gamma = 1, 2, 128, 1000, 700, 64, 0.25, 0.2
    Qn, Kn, Vn = make_inputs(B, H, d, Ns, Nc, seed=13, dtype="bf16")
    Q, K, V = (device_tensor(t, "bf16") for t in (Qn, Kn, Vn))
    O, _, _ = isa.attention_fp8(Q, K, V, b, rho, gamma)
    O2, _, _ = isa.attention_fp8(_token_major(Q), _padded_rows(K), _token_major(V), b, rho, gamma,
                                 out=_token_major(torch.zeros_like(Q)))
    torch.cuda.synchronize()
    assert torch.equal(O, O2)


def test_binding_rejects_mismatched_tensors_before_launch():
    """Shapes, dtypes, devices and outputs are checked before the C-ABI is
    called, so a short V or a small out= never reaches a kernel."""
    Qn, Kn, Vn = make_inputs(1, 2, 64, 300, 200, seed=1, dtype="bf16")
    Q, K, V = (device_tensor(t, "bf16") for t in (Qn, Kn, Vn))
    with pytest.raises(ValueError):
        isa.attention(Q, K, V[:, :, :400], 16, 0.5, 0.5)          # V shorter than K
    with pytest.raises(ValueError):
        isa.attention(Q, K, V.float(), 16, 0.5, 0.5)              # dtype
    with pytest.raises(ValueError):
        isa.attention(Q, K, V, 16, 0.5, 0.5, out=torch.empty((1, 2, 299, 64), dtype=Q.dtype, device="cuda"))
    with pytest.raises(ValueError):
        isa.attention(Q, K, V, 16, 0.5, 0.5, out=torch.empty((1, 2, 300, 64), dtype=Q.dtype))   # host tensor
    with pytest.raises(ValueError):
        isa.attention(Q, K, V, 16, 0.5, 0.5, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        isa.attention(Q, K, V, 16, 0.5, 0.5, workspace=torch.empty(1 << 20, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        isa.attention(Q, K[:, :1], V[:, :1], 16, 0.5, 0.5)        # heads differ
