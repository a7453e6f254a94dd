"""GPU parity where the decay is strong.  The pages put no floor under alpha (blog on Gated
DeltaNet-2, section "Independent control on two axes"), so every decay the rule admits must give
the oracle's results.  The chunk form factors the decay between two tokens of a chunk as
exp(G_i) exp(-G_j), which leaves fp32 range once a channel decays by more than about exp(-64)
over a chunk; the factor kernel flags such chunks and an exact pass recomputes their intra-chunk
products with the pairwise decay (forward and backward).  Checked here, against the fp64 oracle
at the usual tolerances (1e-4 fp32, 3e-3 bf16 forward; 5e-3 gradients):

* log alpha = -2 on every token (-128 per chunk: every chunk flagged);
* log alpha = log sigmoid(N(-2, 1)) (about -150 per chunk);
* one token at -100, and one token at -inf (alpha = 0) in half the channels, in otherwise
  ordinary decay (the per-token floor of -30 keeps those chunks on the fast path);
* -2 over one chunk of one head only, so that one call holds flagged and unflagged chunks;
* bf16 logit gates with x_a = N(-4, 0.5) (about -257 per chunk);
* log alpha about -0.95 per token (-59 to -63 per chunk: unflagged, the fast path at its edge,
  where exp(-G) reaches 1e27).

Each case runs the inference forward, the one-call backward and the staged training chain
(factors, both sweeps, token gradients) and checks which chunks were flagged.  The shapes cover
the wide sweep (bf16, dk 128), the four-wave sweep (fp32, dk 32 and 64), the segmented forward
and backward (one head, 65 chunks) and the one-launch sweeps."""
import numpy as np
import pytest
import torch

import oracle
import linear_attention_sequence_gdn2_amd as gdn2
from linear_attention_sequence_gdn2_amd.inputs import make_inputs
from _util import flags_bytes, oracle_args, rel_err, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 3e-3}
NAMES = ["dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0"]
# a chunk is flagged when some channel's decay over it falls below 2^-92 (natural log -63.77)
FLAG_LOG = -92.0 * np.log(2.0)


def _oracle_inputs(inp):
    if inp.get("gate_logits"):
        return [inp["q32"], inp["k32"], inp["v32"], *oracle.gates_from_logits(inp["log_alpha"], inp["b"], inp["w"]),
                inp["S0"]]
    return oracle_args(inp)


def _expected_flags(inp, B, T, H):
    """Per chunk (in the kernels' order b, h, c): True where the decay is strong enough to be
    flagged, None where it is too close to the threshold to say (not asserted)."""
    if inp.get("gate_logits"):
        la = oracle.gates_from_logits(inp["log_alpha"], inp["b"], inp["w"])[0]
    else:
        la = inp["log_alpha"].double().numpy()
    la = np.maximum(la, -30.0)                      # the per-token floor of the kernels
    nc = (T + 63) // 64
    out = []
    for b in range(B):
        for h in range(H):
            for c in range(nc):
                tot = la[b, 64 * c:64 * c + 64, h].sum(axis=0).min()
                out.append(None if abs(tot - FLAG_LOG) < 0.1 else bool(tot < FLAG_LOG))
    return out


def _flags(factors, items):
    """The flags the factor kernel wrote: the last bytes of the factor buffer."""
    tail = factors[factors.numel() - flags_bytes(items):]
    return tail[:4 * items].view(torch.int32).cpu().numpy()


CASES = [
    # decay, qkv, B, T, H, dk, dv, extra
    ("const2", "f32", 1, 150, 2, 128, 128, {}),
    ("const2", "bf16", 1, 150, 2, 128, 128, {"s0_std": 0.1}),
    ("const2", "f32", 2, 130, 1, 32, 32, {"s0_std": 0.1}),
    ("const2", "bf16", 1, 150, 2, 64, 128, {}),
    ("logsigmoid_m2", "bf16", 2, 200, 2, 128, 128, {"s0_std": 0.05}),
    ("logsigmoid_m2", "f32", 1, 190, 2, 64, 64, {"s0_std": 0.05}),
    ("spike", "bf16", 1, 200, 2, 128, 128, {"s0_std": 0.1}),
    ("reset", "f32", 1, 200, 2, 64, 64, {"s0_std": 0.1}),
    ("reset", "bf16", 2, 150, 2, 128, 128, {}),
    ("mixed", "bf16", 2, 300, 3, 128, 64, {"s0_std": 0.05}),
    ("mixed", "f32", 1, 300, 2, 128, 128, {}),
    ("strong_logits", "bf16", 1, 150, 2, 128, 128, {"gate_logits": True, "s0_std": 0.05}),
    ("strong", "f32", 1, 150, 2, 128, 128, {"s0_std": 0.1}),
    ("strong", "bf16", 1, 150, 2, 128, 128, {"s0_std": 0.1}),
    # one head, 65 chunks: the forward and the one-call backward take the segmented sweep
    ("const2", "bf16", 1, 64 * 64 + 40, 1, 128, 128, {"s0_std": 0.1}),
    ("mixed", "bf16", 1, 64 * 64 + 40, 1, 128, 128, {"s0_std": 0.1}),
]


@pytest.mark.parametrize("decay,qkv,B,T,H,dk,dv,extra", CASES)
def test_strong_decay(decay, qkv, B, T, H, dk, dv, extra):
    inp = make_inputs(B, T, H, dk, dv, seed=9100 + T + dk + dv + len(decay), qkv_dtype=qkv, decay=decay,
                      grads=True, **extra)
    print("case", decay, qkv, B, T, H, dk, dv, flush=True)
    d = to_dev(inp)
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"])
    o, sf = gdn2.fwd(*args)
    g = gdn2.bwd(*args, d["dO"], d["dS_final"])
    # the staged training chain; the two sweeps in one launch where the shape allows
    factors = gdn2.bwd_factors(d["q"], d["k"], d["log_alpha"], d["b"])
    o2, sf2, states, dstates, dS0 = gdn2.sweeps(factors, d["v"], d["w"], dk, d["S0"], d["dO"], d["dS_final"])
    g2 = gdn2.bwd_grads(*args[:6], d["dO"], states, dstates, factors)
    g2["dS0"] = dS0
    torch.cuda.synchronize()

    items = B * H * ((T + 63) // 64)
    got = _flags(factors, items)
    want = _expected_flags(inp, B, T, H)
    assert set(np.unique(got).tolist()) <= {0, 1}
    wrong = [i for i, x in enumerate(want) if x is not None and bool(got[i]) != x]
    assert not wrong, ("flags", wrong[:8], got[:16])
    print("flagged chunks %d of %d" % (int(got.sum()), items))

    oin = _oracle_inputs(inp)
    o_ref, sf_ref = oracle.fwd(*oin)
    ref = oracle.bwd(*oin, inp["dO"], inp["dS_final"])
    if inp.get("gate_logits"):
        ref = oracle.logit_grads(inp["log_alpha"], inp["b"], inp["w"], ref)
    errs = {"o": rel_err(o, o_ref), "S_final": rel_err(sf, sf_ref),
            "o (staged)": rel_err(o2, o_ref), "S_final (staged)": rel_err(sf2, sf_ref)}
    print(" ".join("%s=%.2e" % kv for kv in errs.items()))
    assert all(e < TOL[qkv] for e in errs.values()), errs
    for name, grads in (("one call", g), ("staged", g2)):
        e = {n: rel_err(grads[n], ref[n]) for n in NAMES}
        print(name, " ".join("%s=%.2e" % kv for kv in e.items()))
        bad = {n: v for n, v in e.items() if not v < 5e-3}
        assert not bad, (name, bad)


def test_ordinary_decay_flags_nothing():
    """The workloads' decay (log sigmoid(N(3,1)), about -5 per chunk) never takes the exact pass."""
    inp = make_inputs(2, 1000, 4, 128, 128, seed=9177)
    d = to_dev(inp)
    factors = gdn2.bwd_factors(d["q"], d["k"], d["log_alpha"], d["b"])
    torch.cuda.synchronize()
    assert int(_flags(factors, 2 * 4 * 16).sum()) == 0
