"""GPU parity with the gates given as bf16 logits (gdn2_gate_dtype BF16_LOGITS).

The kernels form log_alpha = log(sigmoid(x_a)), b = sigmoid(x_b), w = sigmoid(x_w)
themselves and return gradients w.r.t. the logits.  The reference is the fp64
oracle on the same bf16 logits activated in fp64 (oracle.gates_from_logits), with
its gradients taken to the logits by the chain rule (oracle.logit_grads; both
pinned in test_oracle_pins).  Tolerances as for bf16 inputs: 3e-3 forward, 5e-3
gradients (max-norm relative)."""
import pytest
import torch

import oracle
import linear_attention_sequence_gdn2_amd as gdn2
from linear_attention_sequence_gdn2_amd.inputs import WORKLOADS, make_inputs, make_workload
from _util import rel_err, to_dev

pytestmark = pytest.mark.gpu

NAMES = ["dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0"]


def _oracle_inputs(inp):
    la, b, w = oracle.gates_from_logits(inp["log_alpha"], inp["b"], inp["w"])
    return [inp["q32"], inp["k32"], inp["v32"], la, b, w, inp["S0"]]


def _check_fwd(inp, d):
    o, sf = gdn2.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"])
    torch.cuda.synchronize()
    o_ref, sf_ref = oracle.fwd(*_oracle_inputs(inp))
    eo, es = rel_err(o, o_ref), rel_err(sf, sf_ref)
    print("logit gates: o err %.3e  S_final err %.3e" % (eo, es))
    assert eo < 3e-3 and es < 3e-3, (eo, es)


def _check_bwd(inp, d, g):
    xs = (inp["log_alpha"], inp["b"], inp["w"])
    ref = oracle.logit_grads(*xs, oracle.bwd(*_oracle_inputs(inp), inp["dO"], inp["dS_final"]))
    errs = {n: rel_err(g[n], ref[n]) for n in NAMES}
    print(" ".join("%s=%.2e" % kv for kv in errs.items()))
    bad = {n: e for n, e in errs.items() if not e < 5e-3}
    assert not bad, bad


@pytest.mark.parametrize("B,T,H,dk,dv,s0", [
    (1, 1, 1, 32, 32, 0.5),
    (2, 65, 2, 64, 128, 0.3),
    (1, 200, 3, 128, 128, 0.02),
    (2, 130, 1, 128, 32, 0.0),
])
def test_logit_gates_fwd_bwd(B, T, H, dk, dv, s0):
    inp = make_inputs(B, T, H, dk, dv, seed=8000 + T + dk, s0_std=s0, grads=True, gate_logits=True)
    d = to_dev(inp)
    _check_fwd(inp, d)
    g = gdn2.bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], d["dO"], d["dS_final"])
    torch.cuda.synchronize()
    _check_bwd(inp, d, g)


def test_logit_gates_training_workload():
    """The B8 T2048 H16 d128 training shape, staged as in a training step."""
    inp = make_workload(WORKLOADS["logits_bf16_B8H16T2048d128"])
    d = to_dev(inp)
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    o, sf, states = gdn2.fwd_states(*args)
    g = gdn2.bwd_saved(*args, states, d["dO"], d["dS_final"])
    torch.cuda.synchronize()
    o_ref, sf_ref = oracle.fwd(*_oracle_inputs(inp))
    assert rel_err(o, o_ref) < 3e-3 and rel_err(sf, sf_ref) < 3e-3
    _check_bwd(inp, d, g)


def test_logit_gates_decode_step():
    inp = make_inputs(4, 1, 8, 128, 64, seed=8100, s0_std=0.3, gate_logits=True)
    d = to_dev(inp)
    tk = {n: d[n][:, 0].contiguous() for n in ("q", "k", "v", "log_alpha", "b", "w")}
    o, S1 = gdn2.step(tk["q"], tk["k"], tk["v"], tk["log_alpha"], tk["b"], tk["w"], d["S0"])
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.fwd(*_oracle_inputs(inp))
    eo, es = rel_err(o, o_ref[:, 0]), rel_err(S1, s_ref)
    print("logit step: o %.3e S %.3e" % (eo, es))
    assert eo < 1e-5 and es < 1e-5


def test_logits_need_bf16_qkv():
    inp = make_inputs(1, 8, 1, 32, 32, seed=8200, qkv_dtype="f32", gate_logits=True)
    d = to_dev(inp)
    with pytest.raises(TypeError):
        gdn2.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
