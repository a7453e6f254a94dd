"""fp64 CPU oracle for the Gated DeltaNet-2 operator -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It wraps ``gdn2_oracle.c`` (plain C,
double precision, token by token) through ctypes and shares no code with the
HIP library in ``linear_attention_sequence_gdn2_amd``.

The rule it follows (iplexlaw.co.kr blog on Gated DeltaNet-2, section
"Independent control on two axes"; the paper abstract in the OpenAlex record of
arXiv:2605.22791 states the same gate roles): e = b*k on key channels,
z = w*v on value channels, decay S by diag(exp(log_alpha)) first, read
r = S^T e, write S += k (z - r)^T, and the query reads the updated state.

Pins (see tests/test_oracle_pins.py): KDA and Gated DeltaNet reductions,
read-after-write, brute-force transition products, causal linear attention,
pure decay, finite-difference gradients; for the gate helpers and the output
epilogue below, closed forms, invariances and finite differences.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn2_oracle.c")
_LIB = os.path.join(_HERE, "libgdn2_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, baseline x86-64, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.gdn2_oracle_fwd.argtypes = [I, I, I, I, I] + [P] * 9 + [I]
        lib.gdn2_oracle_fwd.restype = I
        lib.gdn2_oracle_bwd.argtypes = [I, I, I, I, I] + [P] * 16 + [I]
        lib.gdn2_oracle_bwd.restype = I
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def fwd(q, k, v, log_alpha, b, w, S0=None, nthreads=None):
    """Token-by-token forward.  Token tensors are [B,T,H,D]; S0 is [B,H,dk,dv] or None.

    Returns (o [B,T,H,dv], S_final [B,H,dk,dv]) as float64 numpy arrays.
    """
    q, k, v, la, bb, ww, s0 = (_f64(t) for t in (q, k, v, log_alpha, b, w, S0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and la.shape == q.shape and bb.shape == q.shape
    assert v.shape == (B, T, H, dv) and ww.shape == v.shape
    if s0 is not None:
        assert s0.shape == (B, H, dk, dv)
    o = np.empty((B, T, H, dv), np.float64)
    sf = np.empty((B, H, dk, dv), np.float64)
    rc = _load().gdn2_oracle_fwd(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(bb),
                                 _ptr(ww), _ptr(s0), _ptr(o), _ptr(sf),
                                 nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("gdn2_oracle_fwd failed (%d)" % rc)
    return o, sf


def bwd(q, k, v, log_alpha, b, w, S0, dO, dS_final=None, nthreads=None):
    """Reverse-mode gradients of sum(dO*o) + sum(dS_final*S_final).

    Returns a dict with dq, dk, dv, dlog_alpha, db, dw (input shapes) and dS0.
    """
    q, k, v, la, bb, ww, s0, do, dsf = (_f64(t) for t in (q, k, v, log_alpha, b, w, S0, dO, dS_final))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert do.shape == (B, T, H, dv)
    out = {
        "dq": np.empty_like(q), "dk": np.empty_like(k), "dv": np.empty_like(v),
        "dlog_alpha": np.empty_like(la), "db": np.empty_like(bb), "dw": np.empty_like(ww),
        "dS0": np.empty((B, H, dk, dv), np.float64),
    }
    rc = _load().gdn2_oracle_bwd(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(bb),
                                 _ptr(ww), _ptr(s0), _ptr(do), _ptr(dsf),
                                 _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                 _ptr(out["dlog_alpha"]), _ptr(out["db"]), _ptr(out["dw"]),
                                 _ptr(out["dS0"]), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("gdn2_oracle_bwd failed (%d)" % rc)
    return out


# ---- gates given as pre-activation logits ----
# The erase and write gates are sigmoid outputs of their own linear projections (blog on
# Gated DeltaNet-2, section "Independent control on two axes"); the decay keeps an fp32
# log form (section "Token path and parallel training").  With logits x_a, x_b, x_w the
# operator's gates are
#     log_alpha = log(sigmoid(x_a)),   b = sigmoid(x_b),   w = sigmoid(x_w),
# and gradients w.r.t. the logits follow by the chain rule:
#     d/dx log(sigmoid(x)) = sigmoid(-x),   d/dx sigmoid(x) = sigmoid(x) (1 - sigmoid(x)).

def _sigmoid(x):
    # exp(log sigmoid(x)): relative accuracy at both tails
    return np.exp(-np.logaddexp(0.0, -x))


def gates_from_logits(x_a, x_b, x_w):
    """(log_alpha, b, w) in float64 from the three logit tensors (any float dtype)."""
    xa, xb, xw = (_f64(t) for t in (x_a, x_b, x_w))
    log_alpha = -np.logaddexp(0.0, -xa)
    return log_alpha, _sigmoid(xb), _sigmoid(xw)


def logit_grads(x_a, x_b, x_w, grads):
    """Gradients w.r.t. the logits from the oracle's gradients w.r.t. the gate values
    (a dict as returned by bwd); returns a new dict with dlog_alpha, db, dw replaced."""
    xa, xb, xw = (_f64(t) for t in (x_a, x_b, x_w))
    sb, sw = _sigmoid(xb), _sigmoid(xw)
    out = dict(grads)
    out["dlog_alpha"] = grads["dlog_alpha"] * _sigmoid(-xa)
    out["db"] = grads["db"] * sb * (1.0 - sb)
    out["dw"] = grads["dw"] * sw * (1.0 - sw)
    return out


# Gates given per token.  The rule's special cases use one value per (batch, token,
# head) for a gate: one beta for both the erase and the write gate (KDA), a scalar
# decay as well (Gated DeltaNet) -- blog on Gated DeltaNet-2, section "Independent
# control on two axes"; the gate ablations replace the erase or the write gate by its
# mean over the channels (same blog, section "Ablations and training throughput").  A
# per-token gate g[b,t,h] is the per-channel gate g[b,t,h] * ones(D); by the chain rule
# its gradient is the sum over the D channels of the per-channel gradient.
SCALAR_DECAY, SCALAR_ERASE, SCALAR_WRITE = 1, 2, 4
_SCALAR_GATES = (("log_alpha", "dlog_alpha", SCALAR_DECAY), ("b", "db", SCALAR_ERASE), ("w", "dw", SCALAR_WRITE))


def gates_per_token(log_alpha, b, w, dk, dv, scalar):
    """Per-channel float64 gates from gates of which those flagged in `scalar`
    (SCALAR_* bits) are [B, T, H] (one value per token)."""
    out = []
    for (name, _, bit), g, d in zip(_SCALAR_GATES, (log_alpha, b, w), (dk, dk, dv)):
        g = _f64(g)
        out.append(np.repeat(g[..., None], d, axis=-1) if scalar & bit else g)
    return tuple(out)


def per_token_grads(grads, scalar):
    """Gradients w.r.t. the per-token gates flagged in `scalar`, from the oracle's
    per-channel gradients (a dict as returned by bwd): summed over the channel axis."""
    out = dict(grads)
    for _, gname, bit in _SCALAR_GATES:
        if scalar & bit:
            out[gname] = grads[gname].sum(axis=-1)
    return out


# Output epilogue.  The operator's output o of each (batch, token, head) goes through an
# RMS normalisation, then an output gate of its own (not the write gate), then the output
# projection (blog on Gated DeltaNet-2, section "Token path and parallel training").  The
# normalisation is taken over the dv value channels of the head, with a learnable
# per-channel weight and a small eps inside the root; the gate is given as values (its
# activation belongs to its projection, as for the other gates); the projection is a
# plain matrix product outside the operator:
#     y = o / sqrt(mean_j o_j^2 + eps) * weight * g
# The gradients are those of this composition (r = 1 / sqrt(mean o^2 + eps), u = o r):
#     dg = dy * u * weight,   dweight = sum over rows of dy * u * g,
#     du = dy * weight * g,   do = r * (du - u * mean_j(du_j u_j)).

def output_fwd(o, g, weight=None, eps=1e-6):
    """y in float64 (same shape as o [..., dv]); weight [dv] or None (ones)."""
    o, g = _f64(o), _f64(g)
    wt = np.ones(o.shape[-1]) if weight is None else _f64(weight)
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o * r * wt * g


def output_bwd(o, g, weight, eps, dy):
    """Gradients of sum(dy * y) w.r.t. o, g and weight (dict do, dg, dweight; float64)."""
    o, g, dy = _f64(o), _f64(g), _f64(dy)
    wt = np.ones(o.shape[-1]) if weight is None else _f64(weight)
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    u = o * r
    du = dy * wt * g
    do = r * (du - u * np.mean(du * u, axis=-1, keepdims=True))
    return {"do": do, "dg": dy * u * wt, "dweight": (dy * u * g).reshape(-1, o.shape[-1]).sum(axis=0)}

