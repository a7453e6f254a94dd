"""GPU parity of the forward with the output epilogue fused (gdn2_chunk_fwd_output).

The operator's output goes through an RMS normalisation over the dv channels of each
(b, t, h) row, a per-channel weight and an output gate of its own (blog on Gated DeltaNet-2,
section "Token path and parallel training").  The fused path keeps o in registers and
exchanges each row's sums of squares between the workgroups that share the row; it must give
the oracle chain's y (oracle.fwd, then oracle.output_fwd on the fp64 o), agree with the
unfused GPU pair (gdn2_chunk_fwd, then gdn2_output_fwd) to rounding, give gdn2_chunk_fwd's
S_final bit for bit, and report no exchange wait that ran out.

Shapes cover each tile arrangement of the fused sweep (value tiles per head: 1, 2 and 4, on
32- and 64-column tiles), ragged T, dk 64 and 128, fp32 and bf16 gates and outputs, a weight or
none, S0, the gate formats (logits, per token), the full-size forward, and shapes that take
the unfused route (fp32 q/k/v; few heads and a long sequence, where the forward segments)."""
import pytest
import torch

import oracle
import linear_attention_sequence_gdn2_amd as gdn2
from linear_attention_sequence_gdn2_amd.inputs import make_inputs, make_output_inputs
from _util import device_cus, oracle_args, rel_err, to_dev

pytestmark = pytest.mark.gpu

EPS = 1e-6


def _oracle_gates(inp, dk, dv):
    if inp.get("gate_logits"):
        return list(oracle.gates_from_logits(inp["log_alpha"], inp["b"], inp["w"]))
    if inp.get("gate_scalar"):
        return list(oracle.gates_per_token(inp["log_alpha"], inp["b"], inp["w"], dk, dv, inp["gate_scalar"]))
    return [inp["log_alpha"], inp["b"], inp["w"]]


def _run(B, T, H, dk, dv, seed, *, qkv="bf16", g_dtype="bf16", y_bf16=False, weight=True, s0=0.1,
         gate_logits=False, gates="channel", token_gates=False, expect_fused=None):
    inp = make_inputs(B, T, H, dk, dv, seed=seed, qkv_dtype=qkv, s0_std=s0, gate_logits=gate_logits, gates=gates,
                      token_gates=token_gates)
    ex = make_output_inputs(B, T, H, dv, seed=seed + 1, g_dtype=g_dtype)
    d = to_dev(inp)
    g = ex["g"].cuda()
    wt = ex["weight"].cuda() if weight else None
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    qd = torch.bfloat16 if qkv == "bf16" else torch.float32
    gd = torch.bfloat16 if gate_logits else torch.float32
    sc = inp.get("gate_scalar", 0) if token_gates else 0
    fused = gdn2.fwd_output_fused(B, T, H, dk, dv, qd, gd, sc)
    print("case B%d T%d H%d dk%d dv%d qkv=%s g=%s y_bf16=%s fused=%s" % (B, T, H, dk, dv, qkv, g_dtype, y_bf16, fused),
          flush=True)
    if expect_fused is not None:
        assert fused == expect_fused
    y, sf, ws = gdn2.fwd_output(*args, g, wt, EPS, d["S0"], out_dtype=torch.bfloat16 if y_bf16 else torch.float32)
    o2, sf2 = gdn2.fwd(*args, d["S0"])
    y2 = gdn2.output_fwd(o2, g, wt, EPS, out_dtype=torch.float32)
    torch.cuda.synchronize()
    if fused:
        assert gdn2.fwd_output_xerr((B, T, H, dk, dv, qd, gd, sc), ws) == 0
    assert torch.equal(sf, sf2)                     # the state path is the plain sweep's
    e_pair = rel_err(y.float(), y2.double().cpu().numpy())
    oa = [inp["q32"], inp["k32"], inp["v32"]] + _oracle_gates(inp, dk, dv) + [inp["S0"]]
    o_ref, _ = oracle.fwd(*oa)
    y_ref = oracle.output_fwd(o_ref, ex["g"], ex["weight"] if weight else None, EPS)
    e = rel_err(y.float(), y_ref)
    print("  y vs oracle %.2e, vs unfused pair %.2e" % (e, e_pair), flush=True)
    tol = (4e-3 if y_bf16 else 3e-3) if qkv == "bf16" else (4e-3 if y_bf16 else 1e-4)
    assert e < tol, e
    assert e_pair < (4e-3 if y_bf16 else 1e-5), e_pair
    return fused


@pytest.mark.parametrize("B,T,H,dk,dv,g_dtype,y_bf16,weight,s0", [
    (2, 130, 2, 128, 128, "bf16", False, True, 0.1),     # 32-column tiles, four per head
    (1, 200, 3, 64, 64, "f32", True, False, 0.0),        # 32-column tiles, two per head, bf16 y
    (2, 100, 40, 64, 128, "bf16", True, True, 0.05),     # 64-column tiles, two per head (cooperative)
    (3, 70, 50, 128, 64, "f32", False, True, 0.1),       # 64-column tiles, one per head
    (1, 1, 4, 128, 128, "bf16", False, True, 0.3),       # a single token
])
def test_fused_forward_output(B, T, H, dk, dv, g_dtype, y_bf16, weight, s0):
    _run(B, T, H, dk, dv, 9700 + T + H, g_dtype=g_dtype, y_bf16=y_bf16, weight=weight, s0=s0, expect_fused=True)


def test_fused_forward_output_gate_formats():
    _run(2, 150, 3, 128, 128, 9750, gate_logits=True, expect_fused=True)
    _run(2, 150, 3, 64, 128, 9760, gates="gdn", token_gates=True, expect_fused=True)


def test_forward_output_unfused_routes():
    # fp32 q/k/v take the four-wave sweep; few heads and a long sequence segment the forward
    _run(1, 130, 2, 64, 64, 9770, qkv="f32", expect_fused=False)
    _run(1, 64 * 64 + 5, 2, 64, 64, 9780, expect_fused=False)


def test_fused_forward_output_full_size():
    """B8 T2048 H16 dk=dv=128: the configuration of the benchmark's forward (cooperative
    launch of 256 workgroups of 64 columns, two per head)."""
    if device_cus() < 256:
        pytest.skip("the full-size fused launch needs 256 resident workgroups")
    _run(8, 2048, 16, 128, 128, 9790, g_dtype="bf16", y_bf16=True, s0=0.0, expect_fused=True)


def test_fused_forward_output_repeatable():
    """Two calls reuse one workspace (its exchange area is cleared by every call) and give the
    same bits."""
    inp = make_inputs(2, 300, 40, 64, 128, seed=9800, s0_std=0.1)
    ex = make_output_inputs(2, 300, 40, 128, seed=9801, g_dtype="bf16")
    d = to_dev(inp)
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    g, wt = ex["g"].cuda(), ex["weight"].cuda()
    y1, s1, ws = gdn2.fwd_output(*args, g, wt, EPS, d["S0"])
    y2, s2, _ = gdn2.fwd_output(*args, g, wt, EPS, d["S0"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(s1, s2)
