"""GPU parity of the segmented inference forward: with so few heads that the wide sweep would
keep at most one CU in four busy, gdn2_chunk_fwd splits each sequence into segments swept side
by side.  It sweeps every segment's state map from zero and identity starts, composes the maps
in order (S_{s+1} = M_s S_s + N_s) and sweeps again from the true start states.  Checked against
the fp64 oracle (3e-3, bf16) and against the unsegmented factored sweep (1e-3) on ragged T, with
and without S0, both key widths and every gate format.  The one-call backward (gdn2_chunk_bwd)
splits its state sweep the same way: its gradients are checked against the oracle's (5e-3), for
every gate format, and against the unsegmented chain of entry points (1e-3)."""
import ctypes

import pytest
import torch

import oracle
import linear_attention_sequence_gdn2_amd as gdn2
from linear_attention_sequence_gdn2_amd.inputs import make_inputs
from _util import device_cus, flags_bytes, oracle_args, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _oracle_inputs(inp):
    if inp.get("gate_logits"):
        return [inp["q32"], inp["k32"], inp["v32"], *oracle.gates_from_logits(inp["log_alpha"], inp["b"], inp["w"]),
                inp["S0"]]
    if inp.get("gate_scalar"):
        dk, dv = inp["q"].shape[-1], inp["v"].shape[-1]
        return [inp["q32"], inp["k32"], inp["v32"],
                *oracle.gates_per_token(inp["log_alpha"], inp["b"], inp["w"], dk, dv, inp["gate_scalar"]), inp["S0"]]
    return oracle_args(inp)


@pytest.mark.parametrize("B,T,H,dk,dv,extra", [
    (1, 64 * 70 + 17, 2, 128, 128, {"s0_std": 0.2}),   # 71 chunks: 8 segments of 9, ragged tail
    (1, 64 * 70 + 17, 2, 128, 128, {}),                 # zero start state
    (1, 64 * 64, 4, 64, 128, {"s0_std": 0.1}),          # dk = 64: 8 segments of 8
    (2, 64 * 80, 1, 128, 64, {"s0_std": 0.1}),          # dv = 64, two sequences
    (2, 64 * 64 + 5, 16, 128, 128, {"s0_std": 0.1}),    # a quarter of the CUs: 4 segments of 17
    (1, 64 * 72, 2, 128, 128, {"gate_logits": True, "s0_std": 0.1}),
    (1, 64 * 72, 2, 128, 128, {"gates": "gdn", "token_gates": True, "s0_std": 0.1}),
])
def test_segmented_forward(B, T, H, dk, dv, extra):
    # the shape takes the segmented path: the workspace holds the records, then every segment's
    # [N | M] block and start state
    s = gdn2.make_shape(B, T, H, dk, dv, torch.bfloat16, torch.bfloat16 if extra.get("gate_logits") else torch.float32,
                        7 if extra.get("token_gates") else 0)
    nc = (T + 63) // 64
    rec = 6 * 64 * dk * 2 + 2 * 64 * 64 * 2 + 2 * 16 * 64 * 16 + 4 * dk * 4 + dk * 4
    rec = (rec + 255) // 256 * 256
    cus = device_cus()
    assert B * H * (dv // 64) * 4 <= cus, "the shape is meant to take the segmented path"
    nseg = -(-nc // -(-nc // min(cus // (B * H * dv // 64), nc // 8)))
    seg_bytes = B * H * nseg * dk * ((dv + dk) + dv) * 4
    assert gdn2.load().gdn2_chunk_fwd_workspace_size(ctypes.byref(s)) == \
        B * H * nc * rec + flags_bytes(B * H * nc) + seg_bytes
    inp = make_inputs(B, T, H, dk, dv, seed=9300 + T + dk + dv, **extra)
    d = to_dev(inp)
    o, sf = gdn2.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"])
    factors = gdn2.bwd_factors(d["q"], d["k"], d["log_alpha"], d["b"])
    o2, sf2, _ = gdn2.fwd_factored(factors, d["v"], d["w"], dk, d["S0"], want_states=False)
    torch.cuda.synchronize()
    o_ref, sf_ref = oracle.fwd(*_oracle_inputs(inp))
    eo, es = rel_err(o, o_ref), rel_err(sf, sf_ref)
    print("segmented: o %.2e S_final %.2e" % (eo, es))
    assert eo < 3e-3 and es < 3e-3, (eo, es)
    for x, y in ((o, o2), (sf, sf2)):
        assert float((x - y).abs().max()) <= 1e-3 * float(y.abs().max())


NAMES = ["dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0"]


@pytest.mark.parametrize("B,T,H,dk,dv,extra", [
    (1, 64 * 70 + 17, 2, 128, 128, {"s0_std": 0.2}),   # 8 segments of 9, ragged tail
    (1, 64 * 64, 4, 64, 128, {}),                       # dk = 64, zero start state
    (2, 64 * 64 + 5, 16, 128, 128, {"s0_std": 0.1}),    # a quarter of the CUs: 4 segments of 17
    (1, 64 * 72, 2, 128, 128, {"gate_logits": True, "s0_std": 0.1}),
    (1, 64 * 72, 2, 128, 128, {"gates": "gdn", "token_gates": True, "s0_std": 0.1}),
])
def test_segmented_backward(B, T, H, dk, dv, extra):
    inp = make_inputs(B, T, H, dk, dv, seed=9400 + T + dk + dv, grads=True, **extra)
    d = to_dev(inp)
    g = gdn2.bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], d["dO"], d["dS_final"])
    # the same gradients from the entry points one by one, with the unsegmented state sweep
    factors = gdn2.bwd_factors(d["q"], d["k"], d["log_alpha"], d["b"])
    _, _, states = gdn2.fwd_factored(factors, d["v"], d["w"], dk, d["S0"], want_o=False)
    dstates, dS0 = gdn2.bwd_reverse(factors, d["dO"], dk, d["dS_final"])
    g2 = gdn2.bwd_grads(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["dO"], states, dstates, factors)
    g2["dS0"] = dS0
    torch.cuda.synchronize()
    for n in NAMES:
        x, y = g[n], g2[n]
        assert float((x - y).abs().max()) <= 1e-3 * float(y.abs().max()), n
    # the oracle's gradients, taken to the logits or summed over a per-token gate's channels
    ref = oracle.bwd(*_oracle_inputs(inp), inp["dO"], inp["dS_final"])
    if extra.get("gate_logits"):
        ref = oracle.logit_grads(inp["log_alpha"], inp["b"], inp["w"], ref)
    elif extra.get("token_gates"):
        ref = oracle.per_token_grads(ref, inp["gate_scalar"])
    errs = {n: rel_err(g[n], ref[n]) for n in NAMES}
    print(" ".join("%s=%.2e" % kv for kv in errs.items()))
    bad = {n: e for n, e in errs.items() if not e < 5e-3}
    assert not bad, bad
