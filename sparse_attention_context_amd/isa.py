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
           "isa_run_fp8_stage", "isa_attention_noalloc", "isa_status_string", "isa_last_error",
           "isa_noalloc_scratch_bytes", "isa_trace_read"]

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


class Strides(ctypes.Structure):
    """isa_strides: element strides of the batch, head and row dimensions."""
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("n", ctypes.c_int64)]


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Ns", ctypes.c_int32), ("Nc", ctypes.c_int32),
                ("d", ctypes.c_int32), ("b", ctypes.c_int32), ("rho", ctypes.c_double),
                ("gamma", ctypes.c_double), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("q", Strides), ("k", Strides), ("v", Strides), ("o", Strides)]


class Counts(ctypes.Structure):
    _fields_ = [("nb_s", ctypes.c_int32), ("nb_c", ctypes.c_int32), ("kc", ctypes.c_int32),
                ("kq", ctypes.c_int32), ("m_kept", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("full_keys", ctypes.c_int64)]


class PlanView(ctypes.Structure):
    _fields_ = [("qbar", ctypes.c_void_p), ("kbar", ctypes.c_void_p), ("vbar", ctypes.c_void_p),
                ("sal", ctypes.c_void_p), ("kept_ctx", ctypes.c_void_p), ("sh", ctypes.c_void_p),
                ("full_q", ctypes.c_void_p), ("taylor_q", ctypes.c_void_p), ("counts", Counts)]


class TraceEntry(ctypes.Structure):
    _fields_ = [("stage", ctypes.c_char_p), ("ms", ctypes.c_float)]


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
        L.isa_attention_noalloc.argtypes = [P(Desc), vp, vp, vp, vp, vp]
        L.isa_attention_noalloc.restype = ctypes.c_int
        L.isa_trace_read.argtypes = [ctypes.POINTER(TraceEntry), ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
        L.isa_trace_read.restype = ctypes.c_int
        L.isa_noalloc_scratch_bytes.argtypes = []
        L.isa_noalloc_scratch_bytes.restype = ctypes.c_size_t
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


def _strides(t):
    """(b, h, n) element strides of a [B,H,rows,d] tensor view; None: contiguous."""
    if t is None:
        return None
    return tuple(int(x) for x in t.stride()[:3])


def make_desc(B, H, Ns, Nc, d, b, rho, gamma, dtype, q=None, k=None, v=None, o=None):
    """isa_desc; q, k, v, o: (b, h, n) element strides of each tensor, None for
    contiguous [B,H,rows,d]."""
    dt = {torch.bfloat16: ISA_BF16, torch.float32: ISA_F32, "bf16": ISA_BF16, "f32": ISA_F32}.get(dtype, dtype)
    st = [Strides(*x) if x is not None else Strides(0, 0, 0) for x in (q, k, v, o)]
    return Desc(int(B), int(H), int(Ns), int(Nc), int(d), int(b), float(rho), float(gamma), int(dt), 0, *st)


def desc_for(Q, K, b, rho, gamma, V=None, O=None):
    """Descriptor of Q [B,H,Ns,d], K (and V) [B,H,Ns+Nc,d] and O [B,H,Ns,d]
    (torch tensors or views; their strides go into the descriptor)."""
    B, H, Ns, d = Q.shape
    return make_desc(B, H, Ns, K.shape[2] - Ns, d, b, rho, gamma, Q.dtype, _strides(Q), _strides(K),
                     _strides(V if V is not None else K), _strides(O))


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


def _tensor(name, t, shape, like):
    """t must be a 4-D device tensor (or view) of `shape`, the dtype and
    device of `like`, with a unit-stride last dimension."""
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != like.dtype or t.device != like.device or not t.is_cuda:
        raise ValueError("%s must be a %s tensor on %s" % (name, like.dtype, like.device))
    if t.dim() != 4 or (t.shape[3] > 1 and t.stride(3) != 1):
        raise ValueError("%s must be [B,H,rows,d] with d unit-stride" % name)


def _inputs(Q, K, V):
    """Validates Q [B,H,Ns,d], K and V [B,H,Ns+Nc,d] (device tensors or
    strided views of one dtype); returns (B, H, Ns, Nk, d)."""
    if not isinstance(Q, torch.Tensor) or Q.dim() != 4 or not Q.is_cuda:
        raise ValueError("Q must be a [B,H,Ns,d] device tensor")
    if not isinstance(K, torch.Tensor) or K.dim() != 4:
        raise ValueError("K must be a [B,H,Ns+Nc,d] device tensor")
    B, H, Ns, d = Q.shape
    Nk = K.shape[2]
    if Nk < Ns:
        raise ValueError("K has %d rows, fewer than Q's %d source rows" % (Nk, Ns))
    _tensor("Q", Q, (B, H, Ns, d), Q)
    _tensor("K", K, (B, H, Nk, d), Q)
    _tensor("V", V, (B, H, Nk, d), Q)
    return B, H, Ns, Nk, d


def _output(name, t, shape, like):
    """A caller's output tensor (validated), or a new contiguous one."""
    if t is None:
        return torch.empty(shape, dtype=like.dtype, device=like.device)
    _tensor(name, t, shape, like)
    return t


def _workspace(name, ws, like, need):
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.device != like.device:
        raise ValueError("%s must be a uint8 tensor on %s" % (name, like.device))
    if not ws.is_contiguous() or ws.numel() < need:
        raise ValueError("%s must be contiguous with at least %d bytes" % (name, need))
    return ws


def new_workspace(desc, device):
    return torch.empty(workspace_size(desc), dtype=torch.uint8, device=device)


def _ws_for(desc, Q, workspace):
    need = workspace_size(desc)
    if workspace is None:
        return new_workspace(desc, Q.device)
    return _workspace("workspace", workspace, Q, need)


def plan(Q, K, V, b, rho, gamma, workspace=None, stream=None):
    """isa_plan: returns the workspace holding the plan."""
    _inputs(Q, K, V)
    desc = desc_for(Q, K, b, rho, gamma, V=V)
    ws = _ws_for(desc, Q, workspace)
    _check("isa_plan", lib().isa_plan(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V), _ptr(ws),
                                      ws.numel(), _stream(stream)))
    return ws


def forward(Q, K, V, workspace, b, rho, gamma, out=None, stream=None):
    """isa_forward on a planned workspace: returns O."""
    _inputs(Q, K, V)
    O = _output("out", out, Q.shape, Q)
    desc = desc_for(Q, K, b, rho, gamma, V=V, O=O)
    ws = _workspace("workspace", workspace, Q, workspace_size(desc))
    _check("isa_forward", lib().isa_forward(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                            _ptr(ws), ws.numel(), _stream(stream)))
    return O


def attention(Q, K, V, b, rho, gamma, out=None, workspace=None, stream=None):
    """isa_attention (plan + forward in one call): returns (O, workspace).
    Q, K, V (and out) may be strided views, e.g. X.transpose(1, 2) of a
    [B,N,H,d] tensor."""
    _inputs(Q, K, V)
    O = _output("out", out, Q.shape, Q)
    desc = desc_for(Q, K, b, rho, gamma, V=V, O=O)
    ws = _ws_for(desc, Q, workspace)
    _check("isa_attention", lib().isa_attention(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                                _ptr(ws), ws.numel(), _stream(stream)))
    return O, ws


def dense_forward(Q, K, V, out=None, stream=None):
    """isa_dense_forward: dense attention of every source row over every key."""
    _inputs(Q, K, V)
    O = _output("out", out, Q.shape, Q)
    desc = desc_for(Q, K, 1, 1.0, 1.0, V=V, O=O)
    _check("isa_dense_forward", lib().isa_dense_forward(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V),
                                                        _ptr(O), _stream(stream)))
    return O


def context_forward(Qc, K, V, out=None, stream=None):
    """isa_context_forward: dense attention of the context query rows Qc
    [B,H,Nc,d] over all keys K, V [B,H,Ns+Nc,d]; returns Oc."""
    if not isinstance(Qc, torch.Tensor) or Qc.dim() != 4 or not isinstance(K, torch.Tensor) or K.dim() != 4:
        raise ValueError("Qc [B,H,Nc,d] needs K and V [B,H,Ns+Nc,d]")
    B, H, Nc, d = Qc.shape
    Nk = K.shape[2]
    if Nk < Nc:
        raise ValueError("K has %d rows, fewer than Qc's %d context rows" % (Nk, Nc))
    _tensor("Qc", Qc, (B, H, Nc, d), Qc)
    _tensor("K", K, (B, H, Nk, d), Qc)
    _tensor("V", V, (B, H, Nk, d), Qc)
    O = _output("out", out, Qc.shape, Qc)
    desc = make_desc(B, H, Nk - Nc, Nc, d, 1, 1.0, 1.0, Qc.dtype, _strides(Qc), _strides(K), _strides(V),
                     _strides(O))
    _check("isa_context_forward", lib().isa_context_forward(ctypes.byref(desc), _ptr(Qc), _ptr(K), _ptr(V), _ptr(O),
                                                            _stream(stream)))
    return O


def run_stage(stage, Q, K, V, workspace, b, rho, gamma, out=None, stream=None):
    """isa_run_stage: one kernel of the layer (stage name or isa_stage value)."""
    _inputs(Q, K, V)
    if out is not None:
        _tensor("out", out, Q.shape, Q)
    desc = desc_for(Q, K, b, rho, gamma, V=V, O=out)
    ws = _workspace("workspace", workspace, Q, workspace_size(desc))
    code = STAGE[stage] if isinstance(stage, str) else int(stage)
    _check("isa_run_stage", lib().isa_run_stage(ctypes.byref(desc), code, _ptr(Q), _ptr(K), _ptr(V), _ptr(out),
                                                _ptr(ws), ws.numel(), _stream(stream)))
    return out


def plan_views(Q, K, workspace, b, rho, gamma):
    """Tensor views of a planned workspace: dict of device tensors + counts."""
    desc = desc_for(Q, K, b, rho, gamma)
    ws = _workspace("workspace", workspace, Q, workspace_size(desc))
    v = PlanView()
    _check("isa_plan_views", lib().isa_plan_views(ctypes.byref(desc), _ptr(ws), ws.numel(), ctypes.byref(v)))
    c = v.counts
    B, H, _, d = Q.shape
    base = ws.data_ptr()

    def view(ptr, dtype, shape):
        n = 1
        for x in shape:
            n *= x
        esz = torch.empty(0, dtype=dtype).element_size()
        off = ptr - base
        return ws[off:off + n * esz].view(dtype).view(*shape)

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


def _grad(name, t, like):
    """A gradient tensor laid out like `like` (its strides: the descriptor
    has one set of strides per pair): the caller's, checked, or a new one."""
    if t is None:
        return torch.empty_strided(like.shape, like.stride(), dtype=like.dtype, device=like.device)
    _tensor(name, t, like.shape, like)
    if t.stride() != like.stride():
        raise ValueError("%s must have the strides of its tensor (%s)" % (name, like.stride()))
    return t


def _bwd_args(Q, K, V, O, dO, workspace, bwd_workspace, dQ, dK, dV, b, rho, gamma):
    _inputs(Q, K, V)
    _tensor("O", O, Q.shape, Q)
    _tensor("dO", dO, Q.shape, Q)
    if dO.stride() != O.stride():
        raise ValueError("dO must have the strides of O (%s)" % (O.stride(),))
    desc = desc_for(Q, K, b, rho, gamma, V=V, O=O)
    ws = _workspace("workspace", workspace, Q, workspace_size(desc))
    bneed = backward_workspace_size(desc)
    bws = new_backward_workspace(desc, Q.device) if bwd_workspace is None else \
        _workspace("bwd_workspace", bwd_workspace, Q, bneed)
    return desc, ws, bws, _grad("dQ", dQ, Q), _grad("dK", dK, K), _grad("dV", dV, V)


def backward(Q, K, V, O, dO, workspace, b, rho, gamma, bwd_workspace=None, dQ=None, dK=None, dV=None, stream=None):
    """isa_backward: (dQ, dK, dV, bwd_workspace) of the layer planned in `workspace`
    (from attention() or plan() + forward() on the same inputs), O its output.
    dQ, dK, dV have the strides of Q, K, V and dO those of O."""
    desc, ws, bws, dQ, dK, dV = _bwd_args(Q, K, V, O, dO, workspace, bwd_workspace, dQ, dK, dV, b, rho, gamma)
    _check("isa_backward", lib().isa_backward(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO),
                                              _ptr(ws), ws.numel(), _ptr(bws), bws.numel(),
                                              _ptr(dQ), _ptr(dK), _ptr(dV), _stream(stream)))
    return dQ, dK, dV, bws


def run_backward_stage(stage, Q, K, V, O, dO, workspace, bwd_workspace, dQ, dK, dV, b, rho, gamma, stream=None):
    """isa_run_backward_stage: one kernel of the backward pass (name or isa_bwd_stage value)."""
    desc, ws, bws, dQ, dK, dV = _bwd_args(Q, K, V, O, dO, workspace, bwd_workspace, dQ, dK, dV, b, rho, gamma)
    code = BWD_STAGE[stage] if isinstance(stage, str) else int(stage)
    _check("isa_run_backward_stage",
           lib().isa_run_backward_stage(ctypes.byref(desc), code, _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO),
                                        _ptr(ws), ws.numel(), _ptr(bws), bws.numel(), _ptr(dQ), _ptr(dK), _ptr(dV),
                                        _stream(stream)))


FP8_STAGES = ["pack", "full", "full_merge"]


def fp8_workspace_size(desc):
    n = ctypes.c_size_t()
    _check("isa_fp8_workspace_size", lib().isa_fp8_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def attention_fp8(Q, K, V, b, rho, gamma, out=None, workspace=None, fp8_workspace=None, stream=None):
    """isa_attention_fp8: the layer with the full route in e4m3; returns (O, workspace, fp8_workspace)."""
    _inputs(Q, K, V)
    O = _output("out", out, Q.shape, Q)
    desc = desc_for(Q, K, b, rho, gamma, V=V, O=O)
    ws = _ws_for(desc, Q, workspace)
    fneed = fp8_workspace_size(desc)
    fws = torch.empty(fneed, dtype=torch.uint8, device=Q.device) if fp8_workspace is None else \
        _workspace("fp8_workspace", fp8_workspace, Q, fneed)
    _check("isa_attention_fp8", lib().isa_attention_fp8(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                                        _ptr(ws), ws.numel(), _ptr(fws), fws.numel(), _stream(stream)))
    return O, ws, fws


def run_fp8_stage(stage, Q, K, V, workspace, fp8_workspace, b, rho, gamma, out=None, stream=None):
    """isa_run_fp8_stage: one kernel of the FP8 full route (name or isa_fp8_stage value)."""
    _inputs(Q, K, V)
    if out is not None:
        _tensor("out", out, Q.shape, Q)
    desc = desc_for(Q, K, b, rho, gamma, V=V, O=out)
    ws = _workspace("workspace", workspace, Q, workspace_size(desc))
    fws = _workspace("fp8_workspace", fp8_workspace, Q, fp8_workspace_size(desc))
    code = FP8_STAGES.index(stage) if isinstance(stage, str) else int(stage)
    _check("isa_run_fp8_stage", lib().isa_run_fp8_stage(ctypes.byref(desc), code, _ptr(Q), _ptr(K), _ptr(V),
                                                        _ptr(out), _ptr(ws), ws.numel(), _ptr(fws), fws.numel(),
                                                        _stream(stream)))


def trace_read(max_entries=16):
    """isa_trace_read: [(stage, ms), ...] of the last isa_attention call made
    while the ISA_TRACE environment variable was set (the library reads it at
    every call)."""
    out = (TraceEntry * max_entries)()
    n = ctypes.c_int(0)
    _check("isa_trace_read", lib().isa_trace_read(out, max_entries, ctypes.byref(n)))
    return [(out[i].stage.decode(), float(out[i].ms)) for i in range(n.value)]


def noalloc_scratch_bytes():
    """Size of the scratch array isa_attention_noalloc works in."""
    return lib().isa_noalloc_scratch_bytes()


def attention_noalloc(Q, K, V, b, rho, gamma, out=None, stream=None):
    """isa_attention_noalloc: the layer with the library's fixed scratch as its
    workspace (no allocation by the library); returns O.  out=None allocates
    O here, in Python; pass out= to allocate nothing at all."""
    _inputs(Q, K, V)
    O = _output("out", out, Q.shape, Q)
    desc = desc_for(Q, K, b, rho, gamma, V=V, O=O)
    _check("isa_attention_noalloc", lib().isa_attention_noalloc(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V),
                                                                _ptr(O), _stream(stream)))
    return O


class CapturedAttention:
    """One isa_attention call captured in a HIP graph (torch.cuda.CUDAGraph)
    on fixed tensors; replay() runs the captured kernel sequence again on the
    current contents of Q, K, V, writing out and workspace.  The library's
    calls only enqueue kernels (no allocation, synchronisation or memset), so
    the whole layer captures as one graph; a replay costs one launch from the
    host instead of one per kernel."""

    def __init__(self, Q, K, V, b, rho, gamma, out=None, workspace=None):
        _inputs(Q, K, V)
        self.out = _output("out", out, Q.shape, Q)
        desc = desc_for(Q, K, b, rho, gamma, V=V, O=self.out)
        self.workspace = _ws_for(desc, Q, workspace)
        args = (Q, K, V, b, rho, gamma)
        # one eager call on a side stream first (the graph then captures
        # launches of modules that are already loaded)
        cur = torch.cuda.current_stream()
        side = torch.cuda.Stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            attention(*args, out=self.out, workspace=self.workspace)
        cur.wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            attention(*args, out=self.out, workspace=self.workspace)

    def replay(self):
        self.graph.replay()
        return self.out
