"""ctypes binding of libgdn2.so (the C ABI in include/gdn2.h).

Gates (log_alpha, b, w) are fp32 values, or -- as bfloat16 tensors -- pre-activation
logits (log_alpha = log sigmoid, b, w = sigmoid, formed in the kernels; gradients are
then w.r.t. the logits).  An fp32 gate may also be given per token, as a [B, T, H]
tensor without the channel axis (one value for all channels of its axis; with bf16
q/k/v); its gradient then comes back as [B, T, H] as well.

Argument marshalling only: checks dtypes, devices and contiguity, allocates
the outputs and the workspace with torch on the inputs' device, and passes raw
device pointers plus the current HIP stream.  Every step of the operator runs
in the HIP kernels of libgdn2.so; there is no fallback.  If the library has
not been built, or the tensors are not on a GPU, the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDN2_LIBRARY may name another build of the same library (the phase-stamped one, for
# instrumented measurement runs)
LIB_PATH = os.environ.get("GDN2_LIBRARY") or os.path.join(_HERE, "libgdn2.so")

GDN2_F32 = 0
GDN2_BF16 = 1
GDN2_GATES_F32 = 0
GDN2_GATES_BF16_LOGITS = 1
GDN2_SCALAR_DECAY, GDN2_SCALAR_ERASE, GDN2_SCALAR_WRITE = 1, 2, 4
STATUS = {0: "GDN2_OK", 1: "GDN2_ERR_INVALID_ARG", 2: "GDN2_ERR_UNSUPPORTED", 3: "GDN2_ERR_WORKSPACE",
          4: "GDN2_ERR_HIP", 5: "GDN2_ERR_SCRATCH"}
EXPORTS = ["gdn2_chunk_fwd", "gdn2_chunk_fwd_workspace_size", "gdn2_chunk_bwd",
           "gdn2_chunk_bwd_workspace_size", "gdn2_strerror", "gdn2_chunk_states_bytes",
           "gdn2_chunk_factors_bytes", "gdn2_chunk_bwd_factors",
           "gdn2_chunk_bwd_reverse", "gdn2_chunk_bwd_grads", "gdn2_step", "gdn2_output_fwd",
           "gdn2_output_bwd_workspace_size", "gdn2_output_bwd", "gdn2_chunk_fwd_factored",
           "gdn2_chunk_sweeps", "gdn2_chunk_sweeps_fused", "gdn2_chunk_fwd_noalloc",
           "gdn2_chunk_fwd_noalloc_max_bytes", "gdn2_chunk_fwd_output", "gdn2_chunk_fwd_output_workspace_size",
           "gdn2_chunk_fwd_output_fused"]


class Gdn2Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int), ("dk", ctypes.c_int),
                ("dv", ctypes.c_int), ("chunk", ctypes.c_int), ("qkv_dtype", ctypes.c_int),
                ("gate_dtype", ctypes.c_int), ("gate_scalar", ctypes.c_int)]


class Gdn2Error(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (%d): %s" % (STATUS.get(code, "?"), code, msg))
        self.code = code


_lib = None


def load():
    """Load libgdn2.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libgdn2.so is not built (%s); run python -m "
                               "linear_attention_sequence_gdn2_amd.build" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        SP = ctypes.POINTER(Gdn2Shape)
        lib.gdn2_chunk_fwd.argtypes = [SP] + [P] * 9 + [P, ctypes.c_size_t, P]
        lib.gdn2_chunk_fwd.restype = ctypes.c_int
        lib.gdn2_chunk_bwd.argtypes = [SP] + [P] * 16 + [P, ctypes.c_size_t, P]
        lib.gdn2_chunk_bwd.restype = ctypes.c_int
        lib.gdn2_chunk_fwd_noalloc.argtypes = [SP] + [P] * 9 + [P]
        lib.gdn2_chunk_fwd_noalloc.restype = ctypes.c_int
        lib.gdn2_chunk_fwd_noalloc_max_bytes.argtypes = []
        lib.gdn2_chunk_fwd_noalloc_max_bytes.restype = ctypes.c_size_t
        lib.gdn2_chunk_fwd_workspace_size.argtypes = [SP]
        lib.gdn2_chunk_fwd_workspace_size.restype = ctypes.c_size_t
        lib.gdn2_chunk_bwd_workspace_size.argtypes = [SP]
        lib.gdn2_chunk_bwd_workspace_size.restype = ctypes.c_size_t
        lib.gdn2_chunk_states_bytes.argtypes = [SP]
        lib.gdn2_chunk_states_bytes.restype = ctypes.c_size_t
        lib.gdn2_chunk_factors_bytes.argtypes = [SP]
        lib.gdn2_chunk_factors_bytes.restype = ctypes.c_size_t
        lib.gdn2_chunk_bwd_factors.argtypes = [SP] + [P] * 5 + [P]
        lib.gdn2_chunk_bwd_factors.restype = ctypes.c_int
        lib.gdn2_chunk_fwd_factored.argtypes = [SP] + [P] * 7 + [P]
        lib.gdn2_chunk_fwd_factored.restype = ctypes.c_int
        lib.gdn2_chunk_bwd_reverse.argtypes = [SP] + [P] * 5 + [P]
        lib.gdn2_chunk_bwd_reverse.restype = ctypes.c_int
        lib.gdn2_chunk_sweeps.argtypes = [SP] + [P] * 11 + [P]
        lib.gdn2_chunk_sweeps.restype = ctypes.c_int
        lib.gdn2_chunk_sweeps_fused.argtypes = [SP]
        lib.gdn2_chunk_sweeps_fused.restype = ctypes.c_int
        lib.gdn2_chunk_bwd_grads.argtypes = [SP] + [P] * 16 + [P]
        lib.gdn2_chunk_bwd_grads.restype = ctypes.c_int
        lib.gdn2_step.argtypes = [SP] + [P] * 9 + [P]
        lib.gdn2_step.restype = ctypes.c_int
        I, F = ctypes.c_int, ctypes.c_float
        lib.gdn2_output_fwd.argtypes = [SP, P, P, I, P, F, P, I, P]
        lib.gdn2_output_fwd.restype = ctypes.c_int
        lib.gdn2_chunk_fwd_output.argtypes = [SP] + [P] * 8 + [I, P, F, P, I, P, P, ctypes.c_size_t, P]
        lib.gdn2_chunk_fwd_output.restype = ctypes.c_int
        lib.gdn2_chunk_fwd_output_workspace_size.argtypes = [SP]
        lib.gdn2_chunk_fwd_output_workspace_size.restype = ctypes.c_size_t
        lib.gdn2_chunk_fwd_output_fused.argtypes = [SP]
        lib.gdn2_chunk_fwd_output_fused.restype = ctypes.c_int
        lib.gdn2_output_bwd_workspace_size.argtypes = [SP]
        lib.gdn2_output_bwd_workspace_size.restype = ctypes.c_size_t
        lib.gdn2_output_bwd.argtypes = [SP, P, P, I, P, F, P, P, P, P, P, ctypes.c_size_t, P]
        lib.gdn2_output_bwd.restype = ctypes.c_int
        lib.gdn2_strerror.argtypes = [ctypes.c_int]
        lib.gdn2_strerror.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _check(code):
    if code != 0:
        raise Gdn2Error(code, load().gdn2_strerror(code).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def make_shape(B, T, H, dk, dv, qkv_dtype, gate_dtype=torch.float32, gate_scalar=0):
    """Gates given as bf16 tensors are pre-activation logits (gdn2_gate_dtype);
    gate_scalar holds the GDN2_SCALAR_* bits of the gates given per token."""
    return Gdn2Shape(B, T, H, dk, dv, 64, GDN2_BF16 if qkv_dtype == torch.bfloat16 else GDN2_F32,
                     GDN2_GATES_BF16_LOGITS if gate_dtype == torch.bfloat16 else GDN2_GATES_F32, gate_scalar)


_GATE_BITS = (("log_alpha", GDN2_SCALAR_DECAY), ("b", GDN2_SCALAR_ERASE), ("w", GDN2_SCALAR_WRITE))


def _gate_scalar(lead, gates):
    """GDN2_SCALAR_* bits of the gates given per token: shape `lead` ([B,T,H], or [B,H]
    for a step) without the channel axis.  `gates` maps gate name -> tensor."""
    sc = 0
    for name, bit in _GATE_BITS:
        t = gates.get(name)
        if t is not None and tuple(t.shape) == tuple(lead):
            sc |= bit
    return sc


def _gate_shape(name, lead, d, sc):
    bit = dict(_GATE_BITS)[name]
    return tuple(lead) if sc & bit else tuple(lead) + (d,)


def _gate_dtype(q, *gates):
    """fp32 gate values, or bf16 gate logits (all three alike; only with bf16 q/k/v)."""
    gd = gates[0].dtype
    if gd not in (torch.float32, torch.bfloat16) or any(g.dtype != gd for g in gates):
        raise TypeError("gdn2: the gates must all be float32 values or all bfloat16 logits")
    if gd == torch.bfloat16 and q.dtype != torch.bfloat16:
        raise TypeError("gdn2: bfloat16 gate logits need bfloat16 q/k/v")
    return gd


def _validate(q, k, v, log_alpha, b, w, extra=()):
    if not q.is_cuda:
        raise RuntimeError("gdn2: tensors must live on a GPU (HIP device); got %s" % q.device)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("q/k/v must be float32 or bfloat16")
    gd = _gate_dtype(q, log_alpha, b, w)
    sc = _gate_scalar((B, T, H), dict(log_alpha=log_alpha, b=b, w=w))
    for name, t, shp, dt in (("k", k, (B, T, H, dk), q.dtype), ("v", v, (B, T, H, dv), q.dtype),
                             ("log_alpha", log_alpha, _gate_shape("log_alpha", (B, T, H), dk, sc), gd),
                             ("b", b, _gate_shape("b", (B, T, H), dk, sc), gd),
                             ("w", w, _gate_shape("w", (B, T, H), dv, sc), gd)):
        if tuple(t.shape) != shp or t.dtype != dt or t.device != q.device:
            raise ValueError("gdn2: %s has shape %s dtype %s device %s, expected %s %s %s"
                             % (name, tuple(t.shape), t.dtype, t.device, shp, dt, q.device))
    for t in (q, k, v, log_alpha, b, w) + tuple(x for x in extra if x is not None):
        if not t.is_contiguous():
            raise ValueError("gdn2: tensors must be contiguous")
    return B, T, H, dk, dv, sc


def _grad_outputs(B, T, H, dk, dv, sc, dev):
    """Empty fp32 gradient tensors; a per-token gate's gradient is [B,T,H]."""
    out = {n: torch.empty((B, T, H, dk), dtype=torch.float32, device=dev) for n in ("dq", "dk")}
    out["dv"] = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    for gname, name, d in (("log_alpha", "dlog_alpha", dk), ("b", "db", dk), ("w", "dw", dv)):
        out[name] = torch.empty(_gate_shape(gname, (B, T, H), d, sc), dtype=torch.float32, device=dev)
    return out


def fwd(q, k, v, log_alpha, b, w, S0=None, want_state=True):
    """o [B,T,H,dv] fp32 and S_final [B,H,dk,dv] fp32 (None if not wanted)."""
    B, T, H, dk, dv, sc = _validate(q, k, v, log_alpha, b, w, (S0,))
    if S0 is not None and (tuple(S0.shape) != (B, H, dk, dv) or S0.dtype != torch.float32):
        raise ValueError("gdn2: S0 must be float32 [B,H,dk,dv]")
    lib = load()
    shape = make_shape(B, T, H, dk, dv, q.dtype, log_alpha.dtype, sc)
    o = torch.empty((B, T, H, dv), dtype=torch.float32, device=q.device)
    sf = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device) if want_state else None
    ws_bytes = lib.gdn2_chunk_fwd_workspace_size(ctypes.byref(shape))
    if ws_bytes == ctypes.c_size_t(-1).value:
        raise Gdn2Error(2, "unsupported shape")
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    _check(lib.gdn2_chunk_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b),
                              _ptr(w), _ptr(S0), _ptr(o), _ptr(sf), _ptr(ws), ws_bytes, _stream(q.device)))
    return o, sf


def fwd_noalloc(q, k, v, log_alpha, b, w, S0=None, want_state=True, o=None, S_final=None):
    """gdn2_chunk_fwd_noalloc: the forward with the chunk records in the library's static
    scratch (no workspace).  o and S_final may be given (preallocated outputs)."""
    B, T, H, dk, dv, sc = _validate(q, k, v, log_alpha, b, w, (S0,))
    if S0 is not None and (tuple(S0.shape) != (B, H, dk, dv) or S0.dtype != torch.float32):
        raise ValueError("gdn2: S0 must be float32 [B,H,dk,dv]")
    lib = load()
    shape = make_shape(B, T, H, dk, dv, q.dtype, log_alpha.dtype, sc)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=q.device)
    if S_final is None and want_state:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    for t, shp in ((o, (B, T, H, dv)), (S_final, (B, H, dk, dv))):
        if t is not None and (tuple(t.shape) != shp or t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("gdn2: outputs must be contiguous float32 of the output shapes")
    _check(lib.gdn2_chunk_fwd_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b),
                                      _ptr(w), _ptr(S0), _ptr(o), _ptr(S_final), _stream(q.device)))
    return o, S_final


def bwd_workspace_bytes(B, T, H, dk, dv, qkv_dtype, gate_dtype=torch.float32, gate_scalar=0):
    shape = make_shape(B, T, H, dk, dv, qkv_dtype, gate_dtype, gate_scalar)
    return load().gdn2_chunk_bwd_workspace_size(ctypes.byref(shape))


def bwd(q, k, v, log_alpha, b, w, S0, dO, dS_final=None, want_dS0=True, workspace=None):
    """Gradients of sum(dO*o) + sum(dS_final*S_final): dict of fp32 tensors
    dq, dk, dv, dlog_alpha, db, dw (input shapes) and dS0 (or None)."""
    B, T, H, dk, dv, sc = _validate(q, k, v, log_alpha, b, w, (S0, dO, dS_final))
    if tuple(dO.shape) != (B, T, H, dv) or dO.dtype != torch.float32:
        raise ValueError("gdn2: dO must be float32 [B,T,H,dv]")
    for name, t in (("S0", S0), ("dS_final", dS_final)):
        if t is not None and (tuple(t.shape) != (B, H, dk, dv) or t.dtype != torch.float32):
            raise ValueError("gdn2: %s must be float32 [B,H,dk,dv]" % name)
    lib = load()
    shape = make_shape(B, T, H, dk, dv, q.dtype, log_alpha.dtype, sc)
    dev = q.device
    out = _grad_outputs(B, T, H, dk, dv, sc, dev)
    out["dS0"] = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if want_dS0 else None
    ws_bytes = lib.gdn2_chunk_bwd_workspace_size(ctypes.byref(shape))
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _check(lib.gdn2_chunk_bwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
                              _ptr(S0), _ptr(dO), _ptr(dS_final), _ptr(out["dq"]), _ptr(out["dk"]),
                              _ptr(out["dv"]), _ptr(out["dlog_alpha"]), _ptr(out["db"]), _ptr(out["dw"]),
                              _ptr(out["dS0"]), _ptr(workspace), workspace.numel(), _stream(dev)))
    return out


def states_shape(B, T, H, dk, dv):
    return (B, H, (T + 63) // 64, dk, dv)


def fwd_states(q, k, v, log_alpha, b, w, S0=None, want_state=True, states=None):
    """Forward that also returns the chunk-start states [B,H,ceil(T/64),dk,dv] fp32:
    (o, S_final, states), from a factor buffer (bwd_factors, then fwd_factored)."""
    B, T, H, dk, dv, sc = _validate(q, k, v, log_alpha, b, w, (S0,))
    factors = bwd_factors(q, k, log_alpha, b)
    return fwd_factored(factors, v, w, dk, S0, want_o=True, want_state=want_state, states=states)


def chunk_states(k, v, log_alpha, b, w, S0=None, q_dtype=None, states=None):
    """Chunk-start states [B,H,ceil(T/64),dk,dv] only, from a factor buffer (the states do not
    depend on q; k stands in for it)."""
    B, T, H, dk, dv, sc = _validate(k, k, v, log_alpha, b, w, (S0,))
    factors = bwd_factors(k, k, log_alpha, b)
    return fwd_factored(factors, v, w, dk, S0, want_o=False, want_state=False, states=states)[2]


def factors_bytes(B, T, H, dk, dv=None):
    """Bytes of the per-chunk adjoint factor buffer of gdn2_chunk_bwd_factors."""
    shape = make_shape(B, T, H, dk, dv if dv is not None else dk, torch.float32)
    n = load().gdn2_chunk_factors_bytes(ctypes.byref(shape))
    if n == ctypes.c_size_t(-1).value:
        raise Gdn2Error(2, "unsupported shape")
    return n


def bwd_factors(q, k, log_alpha, b, factors=None):
    """Per-chunk adjoint factors of the reverse sweep (one kernel): a uint8 device
    tensor of factors_bytes() bytes, read only by bwd_reverse."""
    B, T, H, dk = q.shape
    gd = _gate_dtype(q, log_alpha, b)
    sc = _gate_scalar((B, T, H), dict(log_alpha=log_alpha, b=b))
    for name, t, shp, dt in (("k", k, (B, T, H, dk), q.dtype),
                             ("log_alpha", log_alpha, _gate_shape("log_alpha", (B, T, H), dk, sc), gd),
                             ("b", b, _gate_shape("b", (B, T, H), dk, sc), gd)):
        if tuple(t.shape) != shp or t.dtype != dt or t.device != q.device:
            raise ValueError("gdn2: %s must be %s %s on %s" % (name, shp, dt, q.device))
    for t in (q, k, log_alpha, b):
        if not t.is_contiguous():
            raise ValueError("gdn2: tensors must be contiguous")
    if not q.is_cuda:
        raise RuntimeError("gdn2: tensors must live on a GPU (HIP device); got %s" % q.device)
    lib = load()
    shape = make_shape(B, T, H, dk, dk, q.dtype, gd, sc)
    need = factors_bytes(B, T, H, dk)
    if factors is None:
        factors = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif factors.numel() * factors.element_size() < need or not factors.is_contiguous():
        raise ValueError("gdn2: factors buffer smaller than %d bytes" % need)
    _check(lib.gdn2_chunk_bwd_factors(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(log_alpha), _ptr(b),
                                      _ptr(factors), _stream(q.device)))
    return factors


def fwd_factored(factors, v, w, dk, S0=None, want_o=True, want_state=True, states=None, want_states=True):
    """Forward sweep from the factor buffer of bwd_factors on the same q, k, log_alpha, b
    (one kernel; q, k, log_alpha, b are not read again): (o or None, S_final or None,
    states or None).  w is fp32 values [B,T,H,dv] or [B,T,H] (per token), or bf16 logits."""
    if not v.is_cuda:
        raise RuntimeError("gdn2: tensors must live on a GPU (HIP device); got %s" % v.device)
    B, T, H, dv = v.shape
    if v.dtype not in (torch.float32, torch.bfloat16) or w.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("gdn2: v must be float32 or bfloat16, w float32 values or bfloat16 logits")
    if w.dtype == torch.bfloat16 and v.dtype != torch.bfloat16:
        raise TypeError("gdn2: bfloat16 gate logits need bfloat16 q/k/v")
    sc = _gate_scalar((B, T, H), dict(w=w))
    if tuple(w.shape) != _gate_shape("w", (B, T, H), dv, sc) or w.device != v.device:
        raise ValueError("gdn2: w has shape %s, expected %s" % (tuple(w.shape), _gate_shape("w", (B, T, H), dv, sc)))
    for t in (v, w, S0):
        if t is not None and not t.is_contiguous():
            raise ValueError("gdn2: tensors must be contiguous")
    if S0 is not None and (tuple(S0.shape) != (B, H, dk, dv) or S0.dtype != torch.float32):
        raise ValueError("gdn2: S0 must be float32 [B,H,dk,dv]")
    if factors.device != v.device or factors.numel() * factors.element_size() < factors_bytes(B, T, H, dk, dv):
        raise ValueError("gdn2: factors buffer does not match the shape")
    if not (want_o or want_states):
        raise ValueError("gdn2: nothing to compute (want_o and want_states are both false)")
    lib = load()
    shape = make_shape(B, T, H, dk, dv, v.dtype, w.dtype, sc)
    o = torch.empty((B, T, H, dv), dtype=torch.float32, device=v.device) if want_o else None
    sf = torch.empty((B, H, dk, dv), dtype=torch.float32, device=v.device) if want_state else None
    if want_states and states is None:
        states = torch.empty(states_shape(B, T, H, dk, dv), dtype=torch.float32, device=v.device)
    if not want_states:
        states = None
    _check(lib.gdn2_chunk_fwd_factored(ctypes.byref(shape), _ptr(factors), _ptr(v), _ptr(w), _ptr(S0), _ptr(o),
                                       _ptr(sf), _ptr(states), _stream(v.device)))
    return o, sf, states


def bwd_reverse(factors, dO, dk, dS_final=None, want_dS0=True, dstates=None):
    """Reverse sweep from the factors of bwd_factors (one kernel): (dstates, dS0)."""
    B, T, H, dv = dO.shape
    if dO.dtype != torch.float32 or not dO.is_contiguous():
        raise ValueError("gdn2: dO must be contiguous float32 [B,T,H,dv]")
    if dS_final is not None and (tuple(dS_final.shape) != (B, H, dk, dv) or dS_final.dtype != torch.float32
                                 or not dS_final.is_contiguous() or dS_final.device != dO.device):
        raise ValueError("gdn2: dS_final must be contiguous float32 [B,H,dk,dv]")
    if factors.device != dO.device or factors.numel() * factors.element_size() < factors_bytes(B, T, H, dk, dv):
        raise ValueError("gdn2: factors buffer does not match the shape")
    lib = load()
    shape = make_shape(B, T, H, dk, dv, torch.float32)
    if dstates is None:
        dstates = torch.empty(states_shape(B, T, H, dk, dv), dtype=torch.float32, device=dO.device)
    dS0 = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dO.device) if want_dS0 else None
    _check(lib.gdn2_chunk_bwd_reverse(ctypes.byref(shape), _ptr(factors), _ptr(dO), _ptr(dS_final),
                                      _ptr(dstates), _ptr(dS0), _stream(dO.device)))
    return dstates, dS0


def sweeps_fused(B, T, H, dk, dv, qkv_dtype=torch.bfloat16):
    """Whether sweeps() runs its two sweeps as one launch for this shape."""
    return load().gdn2_chunk_sweeps_fused(ctypes.byref(make_shape(B, T, H, dk, dv, qkv_dtype))) == 1


def sweeps(factors, v, w, dk, S0, dO, dS_final=None, want_state=True, want_dS0=True, states=None, dstates=None):
    """Both sweeps of the training step from the factor buffer of bwd_factors (gdn2_chunk_sweeps):
    (o, S_final or None, states, dstates, dS0 or None), the results of fwd_factored and
    bwd_reverse.  One launch where sweeps_fused() holds, else two."""
    if not v.is_cuda:
        raise RuntimeError("gdn2: tensors must live on a GPU (HIP device); got %s" % v.device)
    B, T, H, dv = v.shape
    if v.dtype not in (torch.float32, torch.bfloat16) or w.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("gdn2: v must be float32 or bfloat16, w float32 values or bfloat16 logits")
    if w.dtype == torch.bfloat16 and v.dtype != torch.bfloat16:
        raise TypeError("gdn2: bfloat16 gate logits need bfloat16 q/k/v")
    sc = _gate_scalar((B, T, H), dict(w=w))
    if tuple(w.shape) != _gate_shape("w", (B, T, H), dv, sc) or w.device != v.device:
        raise ValueError("gdn2: w has shape %s, expected %s" % (tuple(w.shape), _gate_shape("w", (B, T, H), dv, sc)))
    if tuple(dO.shape) != (B, T, H, dv) or dO.dtype != torch.float32 or dO.device != v.device:
        raise ValueError("gdn2: dO must be float32 [B,T,H,dv]")
    for name, t in (("S0", S0), ("dS_final", dS_final)):
        if t is not None and (tuple(t.shape) != (B, H, dk, dv) or t.dtype != torch.float32 or t.device != v.device):
            raise ValueError("gdn2: %s must be float32 [B,H,dk,dv]" % name)
    for t in (v, w, S0, dO, dS_final):
        if t is not None and not t.is_contiguous():
            raise ValueError("gdn2: tensors must be contiguous")
    if factors.device != v.device or factors.numel() * factors.element_size() < factors_bytes(B, T, H, dk, dv):
        raise ValueError("gdn2: factors buffer does not match the shape")
    lib = load()
    shape = make_shape(B, T, H, dk, dv, v.dtype, w.dtype, sc)
    dev = v.device
    o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    sf = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if want_state else None
    if states is None:
        states = torch.empty(states_shape(B, T, H, dk, dv), dtype=torch.float32, device=dev)
    if dstates is None:
        dstates = torch.empty(states_shape(B, T, H, dk, dv), dtype=torch.float32, device=dev)
    dS0 = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if want_dS0 else None
    _check(lib.gdn2_chunk_sweeps(ctypes.byref(shape), _ptr(factors), _ptr(v), _ptr(w), _ptr(S0), _ptr(dO),
                                 _ptr(dS_final), _ptr(o), _ptr(sf), _ptr(states), _ptr(dstates), _ptr(dS0),
                                 _stream(dev)))
    return o, sf, states, dstates, dS0


def bwd_grads(q, k, v, log_alpha, b, w, dO, states, dstates, factors):
    """Token gradients from chunk states, end-state gradients and the factor buffer of
    bwd_factors on the same inputs (one kernel)."""
    B, T, H, dk, dv, sc = _validate(q, k, v, log_alpha, b, w, (dO, states, dstates))
    if factors.device != q.device or factors.numel() * factors.element_size() < factors_bytes(B, T, H, dk, dv):
        raise ValueError("gdn2: factors buffer does not match the shape")
    lib = load()
    shape = make_shape(B, T, H, dk, dv, q.dtype, log_alpha.dtype, sc)
    dev = q.device
    out = _grad_outputs(B, T, H, dk, dv, sc, dev)
    _check(lib.gdn2_chunk_bwd_grads(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b),
                                    _ptr(w), _ptr(dO), _ptr(states), _ptr(dstates), _ptr(factors), _ptr(out["dq"]),
                                    _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlog_alpha"]), _ptr(out["db"]),
                                    _ptr(out["dw"]), _stream(dev)))
    return out


def bwd_saved(q, k, v, log_alpha, b, w, states, dO, dS_final=None, want_dS0=True):
    """Backward from the states written by fwd_states: factors, reverse sweep, token gradients."""
    factors = bwd_factors(q, k, log_alpha, b)
    dstates, dS0 = bwd_reverse(factors, dO, q.shape[-1], dS_final, want_dS0)
    out = bwd_grads(q, k, v, log_alpha, b, w, dO, states, dstates, factors)
    out["dS0"] = dS0
    return out


def step(q, k, v, log_alpha, b, w, S=None, out=None, in_place=False):
    """One recurrent step (decode, one kernel): q, k, log_alpha, b [B,H,dk], v, w [B,H,dv]
    (q/k/v fp32 or bf16; gates fp32 values, or bf16 logits with bf16 q/k/v; an fp32
    gate may be [B,H], one value for all its channels, with bf16 q/k/v),
    S [B,H,dk,dv] fp32 or None (zeros).
    Returns (o [B,H,dv] fp32, S_new).  With in_place=True, S is updated in place."""
    if not q.is_cuda:
        raise RuntimeError("gdn2: tensors must live on a GPU (HIP device); got %s" % q.device)
    B, H, dk = q.shape
    dv = v.shape[-1]
    gd = _gate_dtype(q, log_alpha, b, w)
    sc = _gate_scalar((B, H), dict(log_alpha=log_alpha, b=b, w=w))
    for name, t, shp, dt in (("k", k, (B, H, dk), q.dtype), ("v", v, (B, H, dv), q.dtype),
                             ("log_alpha", log_alpha, _gate_shape("log_alpha", (B, H), dk, sc), gd),
                             ("b", b, _gate_shape("b", (B, H), dk, sc), gd),
                             ("w", w, _gate_shape("w", (B, H), dv, sc), gd)):
        if tuple(t.shape) != shp or t.dtype != dt or t.device != q.device or not t.is_contiguous():
            raise ValueError("gdn2: %s must be contiguous %s %s on %s" % (name, shp, dt, q.device))
    if not q.is_contiguous():
        raise ValueError("gdn2: tensors must be contiguous")
    if S is not None and (tuple(S.shape) != (B, H, dk, dv) or S.dtype != torch.float32 or not S.is_contiguous()):
        raise ValueError("gdn2: S must be contiguous float32 [B,H,dk,dv]")
    if in_place and S is None:
        raise ValueError("gdn2: in_place needs a state")
    lib = load()
    shape = make_shape(B, 1, H, dk, dv, q.dtype, gd, sc)
    o = torch.empty((B, H, dv), dtype=torch.float32, device=q.device)
    S_new = S if in_place else (out if out is not None else
                                torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device))
    _check(lib.gdn2_step(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
                         _ptr(S), _ptr(S_new), _ptr(o), _stream(q.device)))
    return o, S_new


def _output_check(o, g, weight, extra=()):
    if not o.is_cuda:
        raise RuntimeError("gdn2: tensors must live on a GPU (HIP device); got %s" % o.device)
    if o.dim() != 4 or o.dtype != torch.float32:
        raise ValueError("gdn2: o must be float32 [B,T,H,dv]")
    if tuple(g.shape) != tuple(o.shape) or g.dtype not in (torch.float32, torch.bfloat16) or g.device != o.device:
        raise ValueError("gdn2: the output gate must be float32 or bfloat16 with the shape of o")
    if weight is not None and (tuple(weight.shape) != (o.shape[-1],) or weight.dtype != torch.float32
                               or weight.device != o.device):
        raise ValueError("gdn2: weight must be float32 [dv]")
    for t in (o, g, weight) + tuple(extra):
        if t is not None and not t.is_contiguous():
            raise ValueError("gdn2: tensors must be contiguous")
    B, T, H, dv = o.shape
    # dk is not used by the epilogue; any supported value keeps the shape valid
    return make_shape(B, T, H, 32, dv, torch.float32), GDN2_BF16 if g.dtype == torch.bfloat16 else GDN2_F32


def output_fwd(o, g, weight=None, eps=1e-6, out_dtype=torch.float32):
    """Output epilogue (one kernel): y = o / sqrt(mean(o^2 over dv) + eps) * weight * g.
    o fp32 [B,T,H,dv]; g output gate values fp32 or bf16, same shape; weight fp32 [dv]
    or None (ones); y has dtype out_dtype (fp32 or bf16)."""
    shape, gdt = _output_check(o, g, weight)
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("gdn2: the epilogue writes float32 or bfloat16")
    y = torch.empty(o.shape, dtype=out_dtype, device=o.device)
    _check(load().gdn2_output_fwd(ctypes.byref(shape), _ptr(o), _ptr(g), gdt, _ptr(weight), float(eps), _ptr(y),
                                  GDN2_BF16 if out_dtype == torch.bfloat16 else GDN2_F32, _stream(o.device)))
    return y


def fwd_output(q, k, v, log_alpha, b, w, g, weight=None, eps=1e-6, S0=None, want_state=True,
               out_dtype=torch.float32, workspace=None):
    """gdn2_chunk_fwd_output: the forward with the output epilogue fused, o never written:
    y = rmsnorm(o) * weight * g per (b, t, h) row (y of dtype out_dtype, fp32 or bf16) and
    S_final.  g: output gate values fp32 or bf16 [B,T,H,dv]; weight fp32 [dv] or None.
    Returns (y, S_final, workspace); the workspace's last 256 bytes hold the exchange
    diagnostic counter (see fwd_output_xerr)."""
    B, T, H, dk, dv, sc = _validate(q, k, v, log_alpha, b, w, (S0, g, weight))
    if S0 is not None and (tuple(S0.shape) != (B, H, dk, dv) or S0.dtype != torch.float32):
        raise ValueError("gdn2: S0 must be float32 [B,H,dk,dv]")
    if tuple(g.shape) != (B, T, H, dv) or g.dtype not in (torch.float32, torch.bfloat16) or g.device != q.device:
        raise ValueError("gdn2: the output gate must be float32 or bfloat16 [B,T,H,dv]")
    if weight is not None and (tuple(weight.shape) != (dv,) or weight.dtype != torch.float32
                               or weight.device != q.device):
        raise ValueError("gdn2: weight must be float32 [dv]")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("gdn2: the epilogue writes float32 or bfloat16")
    lib = load()
    shape = make_shape(B, T, H, dk, dv, q.dtype, log_alpha.dtype, sc)
    y = torch.empty((B, T, H, dv), dtype=out_dtype, device=q.device)
    sf = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device) if want_state else None
    ws_bytes = lib.gdn2_chunk_fwd_output_workspace_size(ctypes.byref(shape))
    if ws_bytes == ctypes.c_size_t(-1).value:
        raise Gdn2Error(2, "unsupported shape")
    if workspace is None or workspace.numel() * workspace.element_size() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.gdn2_chunk_fwd_output(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b),
                                     _ptr(w), _ptr(S0), _ptr(g), GDN2_BF16 if g.dtype == torch.bfloat16 else GDN2_F32,
                                     _ptr(weight), float(eps), _ptr(y),
                                     GDN2_BF16 if out_dtype == torch.bfloat16 else GDN2_F32, _ptr(sf),
                                     _ptr(workspace), nbytes, _stream(q.device)))
    return y, sf, workspace


def fwd_output_fused(B, T, H, dk, dv, qkv_dtype, gate_dtype=torch.float32, gate_scalar=0):
    """Whether gdn2_chunk_fwd_output fuses the epilogue into the sweep for this shape."""
    return bool(load().gdn2_chunk_fwd_output_fused(ctypes.byref(make_shape(B, T, H, dk, dv, qkv_dtype, gate_dtype,
                                                                             gate_scalar))))


def fwd_output_xerr(shape_args, workspace):
    """The fused path's count of exchange waits that ran out (int32 in the workspace's last
    256 bytes, at the offset gdn2_chunk_fwd_output_workspace_size - 256); 0 in a correct run."""
    n = load().gdn2_chunk_fwd_output_workspace_size(ctypes.byref(make_shape(*shape_args)))
    return int(workspace[n - 256:n - 252].view(torch.int32).item())


def output_bwd_workspace_bytes(B, T, H, dv):
    """Bytes of the workspace output_bwd uses for dweight."""
    n = load().gdn2_output_bwd_workspace_size(ctypes.byref(make_shape(B, T, H, 32, dv, torch.float32)))
    if n == ctypes.c_size_t(-1).value:
        raise Gdn2Error(2, "unsupported shape")
    return n


def output_bwd(o, g, weight, eps, dy, want_dweight=True, workspace=None):
    """Backward of the output epilogue for sum(dy * y): dict dO, dg (fp32, the shape of o)
    and dweight (fp32 [dv], or None).  dO is the operator's upstream gradient."""
    shape, gdt = _output_check(o, g, weight, (dy,))
    if tuple(dy.shape) != tuple(o.shape) or dy.dtype != torch.float32 or dy.device != o.device:
        raise ValueError("gdn2: dy must be float32 with the shape of o")
    lib = load()
    dO = torch.empty_like(o)
    dg = torch.empty(o.shape, dtype=torch.float32, device=o.device)
    dweight = torch.empty(o.shape[-1], dtype=torch.float32, device=o.device) if want_dweight else None
    if want_dweight and workspace is None:
        workspace = torch.empty(lib.gdn2_output_bwd_workspace_size(ctypes.byref(shape)), dtype=torch.uint8,
                                device=o.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.gdn2_output_bwd(ctypes.byref(shape), _ptr(o), _ptr(g), gdt, _ptr(weight), float(eps), _ptr(dy),
                               _ptr(dO), _ptr(dg), _ptr(dweight), _ptr(workspace), nbytes, _stream(o.device)))
    return {"dO": dO, "dg": dg, "dweight": dweight}

