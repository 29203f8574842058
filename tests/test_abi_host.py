"""Host-side tests of the C-ABI library: it loads, exports every function
include/isa.h declares, and validates arguments before any device work.
No GPU is touched: every call here returns before enqueuing anything."""

import ctypes
import math
import os
import re

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
