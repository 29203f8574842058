"""ctypes binding to libisa.so (include/isa.h): argument marshalling only.

PyTorch supplies device memory (``data_ptr()``) and the stream
(``torch.cuda.current_stream().cuda_stream``); every step of the layer runs
in the library's HIP kernels.  There is no fallback: if the library is not
built, or a call fails, an exception is raised.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libisa.so")

ISA_BF16 = 0
ISA_F32 = 1

STATUS = {0: "ISA_OK", 1: "ISA_ERR_INVALID_ARGUMENT", 2: "ISA_ERR_UNSUPPORTED", 3: "ISA_ERR_WORKSPACE",
          4: "ISA_ERR_DEVICE"}

EXPORTS = ["isa_get_counts", "isa_workspace_size", "isa_plan", "isa_forward", "isa_attention",
           "isa_dense_forward", "isa_run_stage", "isa_plan_views", "isa_backward_workspace_size", "isa_backward",
           "isa_run_backward_stage", "isa_context_forward", "isa_fp8_workspace_size", "isa_attention_fp8",
           "isa_run_fp8_stage", "isa_status_string", "isa_last_error"]

# isa_stage values (include/isa.h)
STAGES = ["pool", "saliency", "select_ctx", "pool_kept_v", "pack", "sharp_taylor", "sharp", "select_q",
          "taylor", "full", "full_merge"]
STAGE = {name: i for i, name in enumerate(STAGES)}
# the stage sequence of isa_attention when some query blocks stay on the Taylor route
ATTENTION_STAGES = ["pool", "saliency", "select_ctx", "pool_kept_v", "pack", "sharp_taylor", "select_q", "full",
                    "full_merge"]
# isa_bwd_stage values, in the order isa_backward runs them
BWD_STAGES = ["delta", "dk_pooled", "dv_pooled", "dkv_reduce", "dk_full", "dv_full", "zero_pruned", "dq_full",
              "dq_merge", "dq_pooled"]
BWD_STAGE = {name: i for i, name in enumerate(BWD_STAGES)}


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Ns", ctypes.c_int32), ("Nc", ctypes.c_int32),
                ("d", ctypes.c_int32), ("b", ctypes.c_int32), ("rho", ctypes.c_double),
                ("gamma", ctypes.c_double), ("dtype", ctypes.c_int32)]


class Counts(ctypes.Structure):
    _fields_ = [("nb_s", ctypes.c_int32), ("nb_c", ctypes.c_int32), ("kc", ctypes.c_int32),
                ("kq", ctypes.c_int32), ("m_kept", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("full_keys", ctypes.c_int64)]


class PlanView(ctypes.Structure):
    _fields_ = [("qbar", ctypes.c_void_p), ("kbar", ctypes.c_void_p), ("vbar", ctypes.c_void_p),
                ("sal", ctypes.c_void_p), ("kept_ctx", ctypes.c_void_p), ("sh", ctypes.c_void_p),
                ("full_q", ctypes.c_void_p), ("taylor_q", ctypes.c_void_p), ("counts", Counts)]


class IsaError(RuntimeError):
    def __init__(self, fn, code, detail=""):
        self.code = code
        super().__init__("%s failed: %s%s" % (fn, STATUS.get(code, code), (" -- " + detail) if detail else ""))


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libisa.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.isa_get_counts.argtypes = [P(Desc), P(Counts)]
        L.isa_workspace_size.argtypes = [P(Desc), P(sz)]
        L.isa_plan.argtypes = [P(Desc), vp, vp, vp, vp, sz, vp]
        L.isa_forward.argtypes = [P(Desc), vp, vp, vp, vp, vp, sz, vp]
        L.isa_attention.argtypes = [P(Desc), vp, vp, vp, vp, vp, sz, vp]
        L.isa_dense_forward.argtypes = [P(Desc), vp, vp, vp, vp, vp]
        L.isa_plan_views.argtypes = [P(Desc), vp, sz, P(PlanView)]
        L.isa_run_stage.argtypes = [P(Desc), ctypes.c_int, vp, vp, vp, vp, vp, sz, vp]
        L.isa_context_forward.argtypes = [P(Desc), vp, vp, vp, vp, vp]
        L.isa_fp8_workspace_size.argtypes = [P(Desc), P(sz)]
        L.isa_attention_fp8.argtypes = [P(Desc), vp, vp, vp, vp, vp, sz, vp, sz, vp]
        L.isa_run_fp8_stage.argtypes = [P(Desc), ctypes.c_int, vp, vp, vp, vp, vp, sz, vp, sz, vp]
        L.isa_backward_workspace_size.argtypes = [P(Desc), P(sz)]
        L.isa_backward.argtypes = [P(Desc), vp, vp, vp, vp, vp, vp, sz, vp, sz, vp, vp, vp, vp]
        L.isa_run_backward_stage.argtypes = [P(Desc), ctypes.c_int, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp, vp, vp,
                                             vp]
        L.isa_status_string.argtypes = [ctypes.c_int]
        L.isa_status_string.restype = ctypes.c_char_p
        L.isa_last_error.argtypes = []
        L.isa_last_error.restype = ctypes.c_char_p
        for fn in EXPORTS[:15]:
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(fn, code):
    if code != 0:
        detail = lib().isa_last_error().decode() if code == 4 else ""
        raise IsaError(fn, code, detail)


def make_desc(B, H, Ns, Nc, d, b, rho, gamma, dtype):
    dt = {torch.bfloat16: ISA_BF16, torch.float32: ISA_F32, "bf16": ISA_BF16, "f32": ISA_F32}.get(dtype, dtype)
    return Desc(int(B), int(H), int(Ns), int(Nc), int(d), int(b), float(rho), float(gamma), int(dt))


def desc_for(Q, K, b, rho, gamma):
    """Descriptor of Q [B,H,Ns,d], K [B,H,Ns+Nc,d] (torch tensors)."""
    B, H, Ns, d = Q.shape
    return make_desc(B, H, Ns, K.shape[2] - Ns, d, b, rho, gamma, Q.dtype)


def counts(desc):
    c = Counts()
    _check("isa_get_counts", lib().isa_get_counts(ctypes.byref(desc), ctypes.byref(c)))
    return c


def workspace_size(desc):
    n = ctypes.c_size_t()
    _check("isa_workspace_size", lib().isa_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _inputs(Q, K, V):
    for t in (Q, K, V):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("Q, K, V must be contiguous device tensors")
    if not (Q.dtype == K.dtype == V.dtype):
        raise ValueError("Q, K, V must share one dtype")


def new_workspace(desc, device):
    return torch.empty(workspace_size(desc), dtype=torch.uint8, device=device)


def plan(Q, K, V, b, rho, gamma, workspace=None, stream=None):
    """isa_plan: returns the workspace holding the plan."""
    _inputs(Q, K, V)
    desc = desc_for(Q, K, b, rho, gamma)
    ws = new_workspace(desc, Q.device) if workspace is None else workspace
    _check("isa_plan", lib().isa_plan(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V), _ptr(ws),
                                      ws.numel(), _stream(stream)))
    return ws


def forward(Q, K, V, workspace, b, rho, gamma, out=None, stream=None):
    """isa_forward on a planned workspace: returns O."""
    _inputs(Q, K, V)
    desc = desc_for(Q, K, b, rho, gamma)
    O = torch.empty_like(Q) if out is None else out
    _check("isa_forward", lib().isa_forward(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                            _ptr(workspace), workspace.numel(), _stream(stream)))
    return O


def attention(Q, K, V, b, rho, gamma, out=None, workspace=None, stream=None):
    """isa_attention (plan + forward in one call): returns (O, workspace)."""
    _inputs(Q, K, V)
    desc = desc_for(Q, K, b, rho, gamma)
    ws = new_workspace(desc, Q.device) if workspace is None else workspace
    O = torch.empty_like(Q) if out is None else out
    _check("isa_attention", lib().isa_attention(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                                _ptr(ws), ws.numel(), _stream(stream)))
    return O, ws


def dense_forward(Q, K, V, out=None, stream=None):
    """isa_dense_forward: dense attention of every source row over every key."""
    _inputs(Q, K, V)
    desc = desc_for(Q, K, 1, 1.0, 1.0)
    O = torch.empty_like(Q) if out is None else out
    _check("isa_dense_forward", lib().isa_dense_forward(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V),
                                                        _ptr(O), _stream(stream)))
    return O


def context_forward(Qc, K, V, out=None, stream=None):
    """isa_context_forward: dense attention of the context query rows Qc
    [B,H,Nc,d] over all keys K, V [B,H,Ns+Nc,d]; returns Oc."""
    B, H, Nc, d = Qc.shape
    if K.shape[:2] != (B, H) or K.shape[3] != d or K.shape[2] < Nc or V.shape != K.shape:
        raise ValueError("Qc [B,H,Nc,d] needs K and V [B,H,Ns+Nc,d]")
    for t in (Qc, K, V):
        if t.dtype != Qc.dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("Qc, K, V must be contiguous device tensors of one dtype")
    desc = make_desc(B, H, K.shape[2] - Nc, Nc, d, 1, 1.0, 1.0, Qc.dtype)
    O = torch.empty_like(Qc) if out is None else out
    _check("isa_context_forward", lib().isa_context_forward(ctypes.byref(desc), _ptr(Qc), _ptr(K), _ptr(V), _ptr(O),
                                                            _stream(stream)))
    return O


def run_stage(stage, Q, K, V, workspace, b, rho, gamma, out=None, stream=None):
    """isa_run_stage: one kernel of the layer (stage name or isa_stage value)."""
    desc = desc_for(Q, K, b, rho, gamma)
    code = STAGE[stage] if isinstance(stage, str) else int(stage)
    _check("isa_run_stage", lib().isa_run_stage(ctypes.byref(desc), code, _ptr(Q), _ptr(K), _ptr(V), _ptr(out),
                                                _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def plan_views(Q, K, workspace, b, rho, gamma):
    """Tensor views of a planned workspace: dict of device tensors + counts."""
    desc = desc_for(Q, K, b, rho, gamma)
    v = PlanView()
    _check("isa_plan_views", lib().isa_plan_views(ctypes.byref(desc), _ptr(workspace), workspace.numel(),
                                                  ctypes.byref(v)))
    c = v.counts
    B, H, _, d = Q.shape
    base = workspace.data_ptr()

    def view(ptr, dtype, shape):
        n = 1
        for s in shape:
            n *= s
        esz = torch.empty(0, dtype=dtype).element_size()
        off = ptr - base
        return workspace[off:off + n * esz].view(dtype).view(*shape)

    return {
        "qbar": view(v.qbar, torch.float32, (B, H, c.nb_s, d)),
        "kbar": view(v.kbar, torch.float32, (B, H, c.nb_s + c.nb_c, d)),
        "vbar": view(v.vbar, torch.float32, (B, H, c.nb_s + c.nb_c, d)),
        "sal": view(v.sal, torch.float64, (B, H, c.nb_c)),
        "kept_ctx": view(v.kept_ctx, torch.int32, (B, H, c.kc)),
        "sh": view(v.sh, torch.float64, (B, H, c.nb_s)),
        "full_q": view(v.full_q, torch.int32, (B, H, c.kq)),
        "taylor_q": view(v.taylor_q, torch.int32, (B, H, c.nb_s - c.kq)),
        "counts": {"nb_s": c.nb_s, "nb_c": c.nb_c, "kc": c.kc, "kq": c.kq, "m_kept": c.m_kept,
                   "full_keys": c.full_keys},
    }


def backward_workspace_size(desc):
    n = ctypes.c_size_t()
    _check("isa_backward_workspace_size", lib().isa_backward_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def new_backward_workspace(desc, device):
    return torch.empty(backward_workspace_size(desc), dtype=torch.uint8, device=device)


def _bwd_args(Q, K, V, O, dO, workspace, bwd_workspace, dQ, dK, dV, b, rho, gamma):
    _inputs(Q, K, V)
    for t in (O, dO):
        if t.shape != Q.shape or t.dtype != Q.dtype or not t.is_contiguous():
            raise ValueError("O and dO must be contiguous and shaped and typed like Q")
    desc = desc_for(Q, K, b, rho, gamma)
    bws = new_backward_workspace(desc, Q.device) if bwd_workspace is None else bwd_workspace
    dQ = torch.empty_like(Q) if dQ is None else dQ
    dK = torch.empty_like(K) if dK is None else dK
    dV = torch.empty_like(V) if dV is None else dV
    return desc, bws, dQ, dK, dV


def backward(Q, K, V, O, dO, workspace, b, rho, gamma, bwd_workspace=None, dQ=None, dK=None, dV=None, stream=None):
    """isa_backward: (dQ, dK, dV, bwd_workspace) of the layer planned in `workspace`
    (from attention() or plan() + forward() on the same inputs), O its output."""
    desc, bws, dQ, dK, dV = _bwd_args(Q, K, V, O, dO, workspace, bwd_workspace, dQ, dK, dV, b, rho, gamma)
    _check("isa_backward", lib().isa_backward(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO),
                                              _ptr(workspace), workspace.numel(), _ptr(bws), bws.numel(),
                                              _ptr(dQ), _ptr(dK), _ptr(dV), _stream(stream)))
    return dQ, dK, dV, bws


def run_backward_stage(stage, Q, K, V, O, dO, workspace, bwd_workspace, dQ, dK, dV, b, rho, gamma, stream=None):
    """isa_run_backward_stage: one kernel of the backward pass (name or isa_bwd_stage value)."""
    desc = desc_for(Q, K, b, rho, gamma)
    code = BWD_STAGE[stage] if isinstance(stage, str) else int(stage)
    _check("isa_run_backward_stage",
           lib().isa_run_backward_stage(ctypes.byref(desc), code, _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO),
                                        _ptr(workspace), workspace.numel(), _ptr(bwd_workspace),
                                        bwd_workspace.numel(), _ptr(dQ), _ptr(dK), _ptr(dV), _stream(stream)))


FP8_STAGES = ["pack", "full", "full_merge"]


def fp8_workspace_size(desc):
    n = ctypes.c_size_t()
    _check("isa_fp8_workspace_size", lib().isa_fp8_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def attention_fp8(Q, K, V, b, rho, gamma, out=None, workspace=None, fp8_workspace=None, stream=None):
    """isa_attention_fp8: the layer with the full route in e4m3; returns (O, workspace, fp8_workspace)."""
    _inputs(Q, K, V)
    desc = desc_for(Q, K, b, rho, gamma)
    ws = new_workspace(desc, Q.device) if workspace is None else workspace
    fws = (torch.empty(fp8_workspace_size(desc), dtype=torch.uint8, device=Q.device)
           if fp8_workspace is None else fp8_workspace)
    O = torch.empty_like(Q) if out is None else out
    _check("isa_attention_fp8", lib().isa_attention_fp8(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                                        _ptr(ws), ws.numel(), _ptr(fws), fws.numel(), _stream(stream)))
    return O, ws, fws


def run_fp8_stage(stage, Q, K, V, workspace, fp8_workspace, b, rho, gamma, out=None, stream=None):
    """isa_run_fp8_stage: one kernel of the FP8 full route (name or isa_fp8_stage value)."""
    desc = desc_for(Q, K, b, rho, gamma)
    code = FP8_STAGES.index(stage) if isinstance(stage, str) else int(stage)
    _check("isa_run_fp8_stage", lib().isa_run_fp8_stage(ctypes.byref(desc), code, _ptr(Q), _ptr(K), _ptr(V), _ptr(out),
                                                        _ptr(workspace), workspace.numel(), _ptr(fp8_workspace),
                                                        fp8_workspace.numel(), _stream(stream)))
