"""GPU parity of the recurrent step gdn2_step (decode, one token per (batch, head)).

Against the fp64 oracle run on one token (the per-token rule itself), and against
the chunked forward: T steps chained through the state give the same outputs and
final state as gdn2_chunk_fwd over the T tokens.  Tolerances are max-norm relative:
1e-4 for fp32 q/k/v, 3e-3 for bf16 (the step itself is fp32 arithmetic)."""
import pytest
import torch

import oracle
import linear_attention_sequence_gdn2_amd as gdn2
from linear_attention_sequence_gdn2_amd.inputs import make_inputs
from _util import oracle_args, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _token(d, t):
    """token t of [B,T,H,D] device tensors as contiguous [B,H,D]"""
    return {k: d[k][:, t].contiguous() for k in ("q", "k", "v", "log_alpha", "b", "w")}


@pytest.mark.parametrize("B,H,dk,dv,qkv,s0", [
    (1, 1, 32, 32, "f32", 0.0),
    (2, 3, 64, 128, "f32", 0.5),
    (3, 2, 128, 64, "bf16", 0.3),
    (4, 16, 128, 128, "bf16", 0.02),
    (2, 2, 32, 64, "f32", 1.0),
])
def test_step_matches_oracle(B, H, dk, dv, qkv, s0):
    inp = make_inputs(B, 1, H, dk, dv, seed=7000 + B + dk + dv, qkv_dtype=qkv, s0_std=s0)
    d = to_dev(inp)
    tk = _token(d, 0)
    o, S1 = gdn2.step(tk["q"], tk["k"], tk["v"], tk["log_alpha"], tk["b"], tk["w"], d["S0"])
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.fwd(*oracle_args(inp))
    eo, es = rel_err(o, o_ref[:, 0]), rel_err(S1, s_ref)
    print("step o err %.3e  S err %.3e" % (eo, es))
    assert eo < 1e-5 and es < 1e-5, (eo, es)


def test_step_in_place_equals_out_of_place():
    inp = make_inputs(2, 1, 4, 128, 128, seed=7101, qkv_dtype="bf16", s0_std=0.5)
    d = to_dev(inp)
    tk = _token(d, 0)
    o1, S1 = gdn2.step(tk["q"], tk["k"], tk["v"], tk["log_alpha"], tk["b"], tk["w"], d["S0"])
    S = d["S0"].clone()
    o2, S2 = gdn2.step(tk["q"], tk["k"], tk["v"], tk["log_alpha"], tk["b"], tk["w"], S, in_place=True)
    torch.cuda.synchronize()
    assert S2.data_ptr() == S.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("T,dk,dv,qkv", [(70, 64, 64, "f32"), (130, 128, 128, "bf16"), (33, 32, 128, "f32")])
def test_chained_steps_equal_chunked_forward(T, dk, dv, qkv):
    inp = make_inputs(2, T, 3, dk, dv, seed=7200 + T, qkv_dtype=qkv, s0_std=0.2)
    d = to_dev(inp)
    o_chunk, sf_chunk = gdn2.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"])
    S = d["S0"].clone()
    outs = []
    for t in range(T):
        tk = _token(d, t)
        o, S = gdn2.step(tk["q"], tk["k"], tk["v"], tk["log_alpha"], tk["b"], tk["w"], S, in_place=True)
        outs.append(o)
    torch.cuda.synchronize()
    o_steps = torch.stack(outs, dim=1)
    o_ref, s_ref = oracle.fwd(*oracle_args(inp))
    e_step, e_chunk = rel_err(o_steps, o_ref), rel_err(o_chunk, o_ref)
    e_state = rel_err(S, s_ref)
    print("steps vs oracle o %.3e S %.3e; chunked vs oracle o %.3e" % (e_step, e_state, e_chunk))
    assert e_step < 1e-5 and e_state < 1e-5
    assert rel_err(o_steps, o_chunk.double().cpu().numpy()) < (1e-4 if qkv == "f32" else 3e-3)
