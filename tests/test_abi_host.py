"""Host-side tests of the C-ABI library: it loads, exports every function
include/isa.h declares, and validates arguments before any device work.
No GPU is touched: every call here returns before enqueuing anything."""

import ctypes
import math
import os
import re
import shutil
import subprocess

import pytest

from oracle.isa_oracle import count_rule
from sparse_attention_context_amd import isa
from sparse_attention_context_amd.configs import ALL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "isa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(isa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = isa.lib()
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert sorted(isa.EXPORTS) == names


def _desc(**kw):
    base = dict(B=1, H=2, Ns=256, Nc=256, d=64, b=16, rho=0.5, gamma=0.25, dtype="f32")
    base.update(kw)
    return isa.make_desc(**base)


@pytest.mark.parametrize("w", ALL, ids=lambda w: w.name)
def test_counts_match_the_count_rule(w):
    c = isa.counts(isa.make_desc(w.B, w.H, w.Ns, w.Nc, w.d, w.b, w.rho, w.gamma, w.dtype))
    nb_s, nb_c = math.ceil(w.Ns / w.b), math.ceil(w.Nc / w.b)
    assert (c.nb_s, c.nb_c) == (nb_s, nb_c)
    assert c.kc == count_rule(w.rho, nb_c)
    assert c.kq == count_rule(w.gamma, nb_s)
    assert c.m_kept == nb_s + c.kc
    for g in w.gammas:
        c2 = isa.counts(isa.make_desc(w.B, w.H, w.Ns, w.Nc, w.d, w.b, w.rho, g, w.dtype))
        assert c2.kq == count_rule(g, nb_s)


def test_fp32_fraction_would_round_differently():
    # 0.2 * 275 is exactly 55 in double; the library takes the fractions as doubles
    c = isa.counts(_desc(Ns=17550, Nc=17550, b=64, rho=0.25, gamma=0.2))
    assert (c.kc, c.kq) == (69, 55)


def test_workspace_size_grows_with_problem():
    a = isa.workspace_size(_desc())
    b = isa.workspace_size(_desc(H=4))
    assert 0 < a < b
    assert a % 256 == 0


@pytest.mark.parametrize("kw,code", [
    (dict(rho=-0.1), 1), (dict(rho=1.5), 1), (dict(gamma=float("nan")), 1), (dict(rho=float("nan")), 1),
    (dict(Ns=0), 1), (dict(Nc=-1), 1), (dict(b=0), 1), (dict(B=0), 1), (dict(H=0), 1),
    (dict(d=96), 2), (dict(d=256), 2), (dict(b=257), 2), (dict(dtype=7), 2),
])
def test_invalid_descriptors(kw, code):
    with pytest.raises(isa.IsaError) as e:
        isa.workspace_size(_desc(**kw))
    assert e.value.code == code


def test_null_and_misaligned_pointers_rejected_before_launch():
    L = isa.lib()
    d = _desc()
    need = isa.workspace_size(d)
    host = ctypes.create_string_buffer(need + 512)
    base = (ctypes.addressof(host) + 255) // 256 * 256
    ws = ctypes.c_void_p(base)
    p = ctypes.c_void_p(base)  # never dereferenced: every call below fails validation
    nul = ctypes.c_void_p(0)
    assert L.isa_plan(ctypes.byref(d), nul, p, p, ws, need, nul) == 1
    assert L.isa_plan(ctypes.byref(d), ctypes.c_void_p(base + 2), p, p, ws, need, nul) == 1
    assert L.isa_plan(ctypes.byref(d), p, p, p, ws, need - 1, nul) == 3
    assert L.isa_plan(ctypes.byref(d), p, p, p, ctypes.c_void_p(base + 16), need, nul) == 3
    assert L.isa_forward(ctypes.byref(d), p, p, p, nul, ws, need, nul) == 1
    assert L.isa_attention(ctypes.byref(d), p, p, p, p, ws, 16, nul) == 3
    assert L.isa_dense_forward(ctypes.byref(d), p, p, p, nul, nul) == 1
    bad = _desc(rho=2.0)
    assert L.isa_attention(ctypes.byref(bad), p, p, p, p, ws, need, nul) == 1


def test_plan_views_point_inside_workspace():
    L = isa.lib()
    d = _desc()
    need = isa.workspace_size(d)
    host = ctypes.create_string_buffer(need + 512)
    base = (ctypes.addressof(host) + 255) // 256 * 256
    v = isa.PlanView()
    assert L.isa_plan_views(ctypes.byref(d), ctypes.c_void_p(base), need, ctypes.byref(v)) == 0
    for name in ("qbar", "kbar", "vbar", "sal", "kept_ctx", "sh", "full_q", "taylor_q"):
        ptr = getattr(v, name)
        assert base <= ptr < base + need, name
    assert v.counts.kc == 8 and v.counts.kq == 4


def test_status_strings():
    L = isa.lib()
    for code in range(5):
        assert L.isa_status_string(code).decode().startswith(isa.STATUS[code])
    assert L.isa_last_error() == b""


def test_backward_validation_before_launch():
    L = isa.lib()
    d = _desc(dtype="bf16")
    need = isa.workspace_size(d)
    bneed = isa.backward_workspace_size(d)
    assert bneed > 0 and bneed % 256 == 0
    host = ctypes.create_string_buffer(need + bneed + 1024)
    base = (ctypes.addressof(host) + 255) // 256 * 256
    ws = ctypes.c_void_p(base)
    bws = ctypes.c_void_p(base + (need + 255) // 256 * 256)
    p = ctypes.c_void_p(base)  # never dereferenced: every call below fails validation
    nul = ctypes.c_void_p(0)
    D = ctypes.byref(d)
    # f32 has no backward
    f = _desc(dtype="f32")
    with pytest.raises(isa.IsaError) as e:
        isa.backward_workspace_size(f)
    assert e.value.code == 2
    assert L.isa_backward(ctypes.byref(f), p, p, p, p, p, ws, need, bws, bneed, p, p, p, nul) == 2
    # null / misaligned tensors, small or misaligned workspaces
    assert L.isa_backward(D, p, p, p, p, nul, ws, need, bws, bneed, p, p, p, nul) == 1
    assert L.isa_backward(D, p, p, p, p, p, ws, need, bws, bneed, p, nul, p, nul) == 1
    assert L.isa_backward(D, p, p, p, p, ctypes.c_void_p(base + 4), ws, need, bws, bneed, p, p, p, nul) == 1
    assert L.isa_backward(D, p, p, p, p, p, ws, need - 1, bws, bneed, p, p, p, nul) == 3
    assert L.isa_backward(D, p, p, p, p, p, ws, need, bws, bneed - 1, p, p, p, nul) == 3
    assert L.isa_backward(D, p, p, p, p, p, ws, need, ctypes.c_void_p(base + 16), bneed, p, p, p, nul) == 3
    assert L.isa_backward(D, p, p, p, p, p, ws, need, nul, bneed, p, p, p, nul) == 1
    assert L.isa_run_backward_stage(D, 10, p, p, p, p, p, ws, need, bws, bneed, p, p, p, nul) == 1
    assert L.isa_run_backward_stage(D, -1, p, p, p, p, p, ws, need, bws, bneed, p, p, p, nul) == 1


def test_backward_workspace_sizes_of_the_workloads():
    for w in ALL:
        if w.dtype != "bf16":
            continue
        d = isa.make_desc(w.B, w.H, w.Ns, w.Nc, w.d, w.b, w.rho, w.gamma, w.dtype)
        assert 0 < isa.backward_workspace_size(d) < 2e9


# ---------------------------------------------------------------------------
# strided tensors (isa_desc.q/.k/.v/.o) and the limits of the kernels'
# addressing, all decided on the host before any launch

def _sdesc(**kw):
    base = dict(B=1, H=4, Ns=300, Nc=200, d=128, b=16, rho=0.5, gamma=0.25, dtype="bf16")
    st = {k: kw.pop(k) for k in ("q", "k", "v", "o") if k in kw}
    base.update(kw)
    return isa.make_desc(**base, **st)


def test_token_major_strides_are_accepted():
    # [B,N,H,d] views: tokens before heads
    H, d, Ns, Nk = 4, 128, 300, 500
    d1 = _sdesc(q=(Ns * H * d, d, H * d), k=(Nk * H * d, d, H * d), v=(Nk * H * d, d, H * d),
                o=(Ns * H * d, d, H * d))
    assert isa.workspace_size(d1) == isa.workspace_size(_sdesc())
    # one fused QKV buffer [B,N,3,H,d]: rows 3*H*d apart
    d2 = _sdesc(Nc=0, q=(Ns * 3 * H * d, d, 3 * H * d), k=(Ns * 3 * H * d, d, 3 * H * d),
                v=(Ns * 3 * H * d, d, 3 * H * d))
    assert isa.workspace_size(d2) > 0


@pytest.mark.parametrize("kw,code", [
    (dict(k=(0, 0, -128)), 1),                    # negative stride
    (dict(k=(500 * 4 * 136, 500 * 136, 130)), 1),  # 260-byte rows: not 16-byte aligned
    (dict(q=(300 * 4 * 128, 12, 128)), 1),         # head stride of 24 bytes
    (dict(o=(300 * 4 * 128, 300 * 128, 64)), 1),   # O rows overlap
    (dict(o=(128, 0, 512)), 1),                    # all heads of O on one range
    (dict(k=(500 * 4 * (1 << 23), 500 * (1 << 23), 1 << 23)), 2),   # row step of 2^24 bytes
    (dict(k=(0, 500 * 5000000, 5000000)), 2),      # a head of K spans over 2^31 bytes
    (dict(B=256, H=256), 2),                       # B*H = 65536
    (dict(Ns=(1 << 24) - 10, Nc=10, d=64), 2),     # Ns + Nc = 2^24
])
def test_bad_strides_and_limits_rejected(kw, code):
    with pytest.raises(isa.IsaError) as e:
        isa.workspace_size(_sdesc(**kw))
    assert e.value.code == code


def test_overlapping_inputs_are_valid_but_not_as_gradients():
    """Q rows that overlap are a valid read-only input, but isa_backward
    writes dQ through Q's strides and must refuse them."""
    d = _sdesc(q=(300 * 4 * 128, 300 * 128, 64))
    need = isa.workspace_size(d)
    bneed = isa.backward_workspace_size(d)
    host = ctypes.create_string_buffer(need + bneed + 1024)
    base = (ctypes.addressof(host) + 255) // 256 * 256
    ws = ctypes.c_void_p(base)
    bws = ctypes.c_void_p(base + (need + 255) // 256 * 256)
    p = ctypes.c_void_p(base)   # never dereferenced: the call fails validation
    nul = ctypes.c_void_p(0)
    L = isa.lib()
    assert L.isa_backward(ctypes.byref(d), p, p, p, p, p, ws, need, bws, bneed, p, p, p, nul) == 1


def test_reserved_field_must_be_zero():
    d = _sdesc()
    d.reserved = 3
    with pytest.raises(isa.IsaError) as e:
        isa.workspace_size(d)
    assert e.value.code == 1


def test_planner_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """tests/host/abi_check.cpp with the planner and the validation code
    (isa_layout.cpp), built by g++ with ASan + UBSan: every workspace slice of
    a grid of descriptors, the output-overlap test against brute force, the
    multiply that replaces the head division, random descriptors."""
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "abi_check")
    src = [os.path.join(ROOT, "sparse_attention_context_amd", "csrc", "isa_layout.cpp"),
           os.path.join(ROOT, "tests", "host", "abi_check.cpp")]
    subprocess.run(["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I" + os.path.join(ROOT, "include")] + src + ["-o", exe], check=True)
    r = subprocess.run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"), capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "abi_check ok" in r.stdout


def test_context_rows_strides_are_checked_against_their_row_count():
    """isa_context_forward's Qc and Oc hold Nc rows: their strides are
    validated for Nc rows (an output whose heads would overlap as Ns rows is
    fine), and overlapping Oc rows are refused before any launch."""
    B, H, Ns, Nc, d = 1, 4, 300, 200, 128
    L = isa.lib()
    host = ctypes.create_string_buffer(4096)
    p = ctypes.c_void_p((ctypes.addressof(host) + 255) // 256 * 256)   # never dereferenced
    nul = ctypes.c_void_p(0)
    bad = isa.make_desc(B, H, Ns, Nc, d, 1, 1.0, 1.0, "bf16", o=(H * Nc * d, Nc * d, 64))
    assert L.isa_context_forward(ctypes.byref(bad), p, p, p, p, nul) == 1
    bad_q = isa.make_desc(B, H, Ns, Nc, d, 1, 1.0, 1.0, "bf16", q=(H * Nc * d, Nc * d, 65))
    assert L.isa_context_forward(ctypes.byref(bad_q), p, p, p, p, nul) == 1
    import torch
    if not torch.cuda.is_available():
        # valid for Nc rows: passes validation and fails only at the launch
        # (no device here)
        ok = isa.make_desc(B, H, Ns, Nc, d, 1, 1.0, 1.0, "bf16", q=(H * Nc * d, Nc * d, d), o=(H * Nc * d, Nc * d, d))
        assert L.isa_context_forward(ctypes.byref(ok), p, p, p, p, nul) == 4


def test_noalloc_entry_point_refuses_layers_beyond_its_scratch():
    """isa_attention_noalloc checks the layer's workspace against its fixed
    scratch before any device call."""
    L = isa.lib()
    assert isa.noalloc_scratch_bytes() == 128 << 20
    big = isa.make_desc(1, 24, 32760, 32760, 128, 64, 0.25, 0.3, "bf16")   # the long clip at gamma 0.3: 235 MiB
    assert isa.workspace_size(big) > isa.noalloc_scratch_bytes()
    host = ctypes.create_string_buffer(4096)
    p = ctypes.c_void_p((ctypes.addressof(host) + 255) // 256 * 256)   # never dereferenced
    nul = ctypes.c_void_p(0)
    assert L.isa_attention_noalloc(ctypes.byref(big), p, p, p, p, nul) == 3
    assert L.isa_attention_noalloc(ctypes.byref(big), p, p, p, nul, nul) == 1
    bad = isa.make_desc(1, 2, 300, 200, 64, 16, 2.0, 0.25, "bf16")
    assert L.isa_attention_noalloc(ctypes.byref(bad), p, p, p, p, nul) == 1


def test_trace_read_without_a_traced_call_is_an_error():
    """isa_trace_read checks its arguments and refuses when no traced call
    has been recorded (this process makes no GPU call)."""
    import ctypes
    L = isa.lib()
    n = ctypes.c_int(7)
    assert L.isa_trace_read(None, 0, None) == 1
    assert L.isa_trace_read(None, 4, ctypes.byref(n)) == 1
    assert L.isa_trace_read(None, -1, ctypes.byref(n)) == 1
    out = (isa.TraceEntry * 4)()
    assert L.isa_trace_read(out, 4, ctypes.byref(n)) == 1 and n.value == 0
