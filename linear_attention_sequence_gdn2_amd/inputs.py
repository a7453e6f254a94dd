"""Seeded synthetic inputs for the GDN-2 operator (shared by tests, bench and smoke).

This module holds only random-number generation and the input recipe; none of
the operator's arithmetic lives here.  Both the HIP path and the fp64 oracle
are fed from the same host tensors it returns.

Recipe (shapes from the Gated DeltaNet-2 pages: 16 heads with 128-dim keys and
values, iplexlaw.co.kr blog section "Experimental comparison"; 64-token chunks,
section "Token path and parallel training"; 2K x 8 and 16K x 1 training shapes,
section "Ablations and training throughput", Figure 2):

* q, k ~ N(0, 1) per channel, then L2-normalised per (batch, token, head) in fp32
  (the pages normalise q and k before the operator), then optionally rounded to
  bf16 (round-to-nearest-even).  v ~ N(0, 1), same rounding.
* log_alpha: ``"softplus"``  -> -softplus(N(0,1)) * 0.1   (tiny fp32 workload)
             ``"logsigmoid"`` -> log(sigmoid(N(3,1)))      (decay ~0.9-0.99)
             ``"strong"``     -> -0.95 + 0.02 N(0,1), clamped to [-0.98, -0.92] (a chunk's
                                 cumulative log-decay between -62.8 and -58.8, just above
                                 the -63.8 below which the kernels take their exact pass)
  Stress recipes for the decay range (the pages put no floor under alpha): ``"const2"``
  -> -2 everywhere (-128 per chunk); ``"logsigmoid_m2"`` -> log(sigmoid(N(-2,1)));
  ``"spike"`` -> log(sigmoid(N(3,1))) with token T // 3 at -100 in every channel;
  ``"reset"`` -> the same with token T // 3 at -inf (alpha = 0) in the even channels;
  ``"mixed"`` -> log(sigmoid(N(3,1))) with -2 over the chunk holding token T // 2 in head 0
  only, so one call holds both kinds of chunk.  With ``gate_logits``, ``decay="strong_logits"``
  draws x_a = N(-4, 0.5) (log(sigmoid) near -4 per token) instead of N(3,1).
* gates ``"channel"``: b = sigmoid(N(0,1)) per key channel, w = sigmoid(N(0,1))
  per value channel.  ``"kda"``: one beta = sigmoid(N(0,1)) per (b,t,h),
  broadcast to b and w.  ``"gdn"``: as ``"kda"`` and log_alpha drawn once per
  (b,t,h) and broadcast over key channels.  The gate ablations (blog section
  "Ablations and training throughput"): ``"erase_mean"`` / ``"write_mean"`` draw as
  ``"channel"`` and replace b (resp. w) by its mean over the channels;
  ``"erase2"`` draws as ``"channel"`` with b = 2 * sigmoid(N(0,1)) in [0, 2].
* ``token_gates=True``: a gate that is one value per (b,t,h) is returned as a
  [B, T, H] tensor instead of being broadcast over its channels, and
  ``gate_scalar`` holds its bits (1 decay, 2 erase, 4 write).
* S0 ~ N(0, s0_std) (zeros when s0_std == 0), dO ~ N(0, 1), dS_final ~ N(0, 0.01).
* ``gate_logits=True`` (channel gates, log-sigmoid decay): the same normal draws are
  returned before their activation, rounded to bf16, as ``x_a`` = N(3,1), ``x_b``,
  ``x_w`` = N(0,1); the gate values are then left to the consumer (the operator forms
  log(sigmoid(x_a)), sigmoid(x_b), sigmoid(x_w) itself).

The second argument of every N(mu, sigma) is a standard deviation.  Draw order
is fixed: q, k, v, log_alpha, b, w, S0, dO, dS_final.
"""
from __future__ import annotations

from dataclasses import dataclass, field, asdict

import torch
import torch.nn.functional as F


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    seed: int
    qkv_dtype: str = "bf16"          # "bf16" or "f32"
    decay: str = "logsigmoid"        # "softplus", "logsigmoid", "strong" or a stress recipe
    gates: str = "channel"           # "channel", "kda" or "gdn"
    s0_std: float = 0.0
    grads: bool = False              # also draw dO and dS_final
    extra: dict = field(default_factory=dict)

    def as_dict(self):
        return asdict(self)


# The five workloads of the operator, named by what they are.
WORKLOADS = {
    "tiny_f32_B1H2T128d32": Workload("tiny_f32_B1H2T128d32", 1, 128, 2, 32, 32, 1001,
                                     qkv_dtype="f32", decay="softplus"),
    "fwd_bf16_B8H16T2048d128": Workload("fwd_bf16_B8H16T2048d128", 8, 2048, 16, 128, 128, 1002),
    # the same batch with the upstream gradients drawn too: one training step (fwd + bwd)
    "train_bf16_B8H16T2048d128": Workload("train_bf16_B8H16T2048d128", 8, 2048, 16, 128, 128, 1002, grads=True),
    "long_bf16_B1H16T16384d128": Workload("long_bf16_B1H16T16384d128", 1, 16384, 16, 128, 128, 1003,
                                          s0_std=0.02),
    "kda_bf16_B4H16T4096d128": Workload("kda_bf16_B4H16T4096d128", 4, 4096, 16, 128, 128, 1004,
                                        gates="kda"),
    "gdn_bf16_B4H16T4096d128": Workload("gdn_bf16_B4H16T4096d128", 4, 4096, 16, 128, 128, 1004,
                                        gates="gdn"),
    "fwdbwd_bf16_B4H16T4096d128": Workload("fwdbwd_bf16_B4H16T4096d128", 4, 4096, 16, 128, 128, 1005,
                                           s0_std=0.02, grads=True),
    # the training shape with the gates given as bf16 logits (activated in the kernels)
    "logits_bf16_B8H16T2048d128": Workload("logits_bf16_B8H16T2048d128", 8, 2048, 16, 128, 128, 1006,
                                           grads=True, extra={"gate_logits": True}),
    # the training shape with Gated DeltaNet's gates given once per token ([B,T,H])
    "gdn_token_bf16_B8H16T2048d128": Workload("gdn_token_bf16_B8H16T2048d128", 8, 2048, 16, 128, 128, 1007,
                                              gates="gdn", grads=True, extra={"token_gates": True}),
}


def make_inputs(B, T, H, dk, dv, seed, *, qkv_dtype="bf16", decay="logsigmoid", gates="channel",
                s0_std=0.0, grads=False, gate_logits=False, token_gates=False):
    """Return a dict of CPU tensors.

    ``q``, ``k``, ``v`` have dtype bf16 (or fp32 when ``qkv_dtype == "f32"``);
    ``q32``, ``k32``, ``v32`` are the same values widened exactly to fp32.
    Gates, decay, states and upstream gradients are fp32.
    """
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    shp_k = (B, T, H, dk)
    shp_v = (B, T, H, dv)

    def randn(*shape):
        return torch.randn(*shape, generator=g, dtype=torch.float32)

    q = randn(*shp_k)
    q = q / q.norm(dim=-1, keepdim=True).clamp_min(1e-30)
    k = randn(*shp_k)
    k = k / k.norm(dim=-1, keepdim=True).clamp_min(1e-30)
    v = randn(*shp_v)

    if gate_logits:
        if gates != "channel" or decay not in ("logsigmoid", "strong_logits"):
            raise ValueError("gate logits are drawn for channel gates with a log-sigmoid decay")
        x_a = (randn(*shp_k) + 3.0 if decay == "logsigmoid" else randn(*shp_k) * 0.5 - 4.0).to(torch.bfloat16)
        x_b = randn(*shp_k).to(torch.bfloat16)
        x_w = randn(*shp_v).to(torch.bfloat16)
    if gate_logits:
        la = b = w = None
    elif gates == "gdn":
        la = F.logsigmoid(randn(B, T, H, 1) + 3.0).expand(shp_k).contiguous()
    elif decay == "softplus":
        la = -F.softplus(randn(*shp_k)) * 0.1
    elif decay == "logsigmoid":
        la = F.logsigmoid(randn(*shp_k) + 3.0)
    elif decay == "strong":
        # about -0.95 per token: a 64-token chunk sums to between -62.8 and -58.8
        la = (-0.95 + 0.02 * randn(*shp_k)).clamp(-0.98, -0.92)
    elif decay == "const2":
        la = randn(*shp_k) * 0.0 - 2.0
    elif decay == "logsigmoid_m2":
        la = F.logsigmoid(randn(*shp_k) - 2.0)
    elif decay in ("spike", "reset", "mixed"):
        la = F.logsigmoid(randn(*shp_k) + 3.0)
        if decay == "spike":
            la[:, T // 3] = -100.0
        elif decay == "reset":
            la[:, T // 3, :, 0::2] = float("-inf")
        else:
            c0 = (T // 2) // 64 * 64
            la[:, c0:c0 + 64, 0] = -2.0
    else:
        raise ValueError(decay)

    if gate_logits:
        pass
    elif gates in ("channel", "erase_mean", "write_mean", "erase2"):
        b = torch.sigmoid(randn(*shp_k))
        w = torch.sigmoid(randn(*shp_v))
        if gates == "erase_mean":
            b = b.mean(dim=-1, keepdim=True).expand(shp_k).contiguous()
        elif gates == "write_mean":
            w = w.mean(dim=-1, keepdim=True).expand(shp_v).contiguous()
        elif gates == "erase2":
            b = 2.0 * b
    elif gates in ("kda", "gdn"):
        beta = torch.sigmoid(randn(B, T, H, 1))
        b = beta.expand(shp_k).contiguous()
        w = beta.expand(shp_v).contiguous()
    else:
        raise ValueError(gates)
    scalar = 0
    if token_gates:
        if gate_logits:
            raise ValueError("per-token gates are fp32 values")
        scalar = {"gdn": 7, "kda": 6, "erase_mean": 2, "write_mean": 4}.get(gates, 0)
        if scalar & 1:
            la = la[..., 0]
        if scalar & 2:
            b = b[..., 0]
        if scalar & 4:
            w = w[..., 0]

    if s0_std > 0:
        S0 = randn(B, H, dk, dv) * s0_std
    else:
        S0 = None

    out = {}
    if qkv_dtype == "bf16":
        for name, t in (("q", q), ("k", k), ("v", v)):
            tb = t.to(torch.bfloat16)
            out[name] = tb
            out[name + "32"] = tb.float()
    elif qkv_dtype == "f32":
        for name, t in (("q", q), ("k", k), ("v", v)):
            out[name] = t
            out[name + "32"] = t
    else:
        raise ValueError(qkv_dtype)
    if gate_logits:
        out.update(log_alpha=x_a.contiguous(), b=x_b.contiguous(), w=x_w.contiguous(), S0=S0, gate_logits=True)
    else:
        out.update(log_alpha=la.contiguous(), b=b.contiguous(), w=w.contiguous(), S0=S0, gate_scalar=scalar)

    if grads:
        out["dO"] = randn(*shp_v)
        out["dS_final"] = randn(B, H, dk, dv) * 0.01
    return out


def make_workload(wl: Workload, **override):
    kw = dict(B=wl.B, T=wl.T, H=wl.H, dk=wl.dk, dv=wl.dv, seed=wl.seed, qkv_dtype=wl.qkv_dtype,
              decay=wl.decay, gates=wl.gates, s0_std=wl.s0_std, grads=wl.grads,
              gate_logits=wl.extra.get("gate_logits", False), token_gates=wl.extra.get("token_gates", False))
    kw.update(override)
    return make_inputs(**kw)


def make_output_inputs(B, T, H, dv, seed, *, g_dtype="f32"):
    """Inputs of the output epilogue (CPU tensors): the operator output o ~ N(0, 0.5) fp32,
    the output gate g = sigmoid(N(0,1)) (fp32, or rounded to bf16 with g_dtype="bf16"),
    the norm weight ~ U(0.5, 1.5) [dv] fp32 and the upstream gradient dy ~ N(0,1) fp32.
    Draw order: o, g, weight, dy."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    o = torch.randn(B, T, H, dv, generator=gen) * 0.5
    g = torch.sigmoid(torch.randn(B, T, H, dv, generator=gen))
    if g_dtype == "bf16":
        g = g.to(torch.bfloat16)
    elif g_dtype != "f32":
        raise ValueError(g_dtype)
    weight = torch.rand(dv, generator=gen) + 0.5
    dy = torch.randn(B, T, H, dv, generator=gen)
    return {"o": o, "g": g, "weight": weight, "dy": dy}


def make_inputs_device(B, T, H, dk, dv, seed, device, *, s0_std=0.0, grads=False, read_after_write=False):
    """The bf16 workload recipe above (channel gates, log(sigmoid(N(3,1))) decay), drawn on
    ``device`` with a seeded device generator: for shapes whose host-side generation would
    take minutes (tensors of several GiB).  The same seed gives the same tensors on the same
    device type; they are not the values make_inputs draws on the host.  Draw order: q, k, v,
    log_alpha, b, w, S0, dO, dS_final.

    ``read_after_write=True`` replaces q and k by one hot key (a uniformly drawn channel per
    (b, t, h), drawn after dS_final) and b by ones: the erase-then-write case of the rule in
    which every output equals w * v of its own token."""
    g = torch.Generator(device=device).manual_seed(int(seed))

    def randn(*shape):
        return torch.randn(*shape, generator=g, dtype=torch.float32, device=device)

    def unit_bf16(shape):
        x = randn(*shape)
        x /= x.norm(dim=-1, keepdim=True).clamp_min(1e-30)
        return x.to(torch.bfloat16)

    out = {"q": unit_bf16((B, T, H, dk)), "k": unit_bf16((B, T, H, dk)),
           "v": randn(B, T, H, dv).to(torch.bfloat16)}
    la = randn(B, T, H, dk)
    la += 3.0
    out["log_alpha"] = F.logsigmoid(la)
    del la
    out["b"] = torch.sigmoid(randn(B, T, H, dk))
    out["w"] = torch.sigmoid(randn(B, T, H, dv))
    out["S0"] = randn(B, H, dk, dv) * s0_std if s0_std > 0 else None
    if grads:
        out["dO"] = randn(B, T, H, dv)
        out["dS_final"] = randn(B, H, dk, dv) * 0.01
    if read_after_write:
        ch = torch.randint(0, dk, (B, T, H), generator=g, device=device)
        onehot = torch.zeros(B, T, H, dk, dtype=torch.bfloat16, device=device)
        onehot.scatter_(-1, ch.unsqueeze(-1), 1.0)
        del ch
        out["q"], out["k"] = onehot, onehot.clone()
        out["b"].fill_(1.0)
    return out
