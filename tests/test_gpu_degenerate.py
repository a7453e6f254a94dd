"""GPU parity at the degenerate gate values of the Gated DeltaNet-2 rule, and an identity of the
rule checked at full size without the oracle.

Degenerate gates (blog on Gated DeltaNet-2, section "Independent control on two axes": b gates
the erase on the key channels, w the write on the value channels, alpha the decay):
  b = 0   no erase: the rule becomes gated linear attention, S = diag(alpha) S + k z^T;
  w = 0   no write: the state only decays and is read;
  alpha = 1 (log_alpha = 0): no decay;
  b = 1   full erase of the key direction (the delta rule).
Forward and backward against the fp64 oracle on the same inputs (1e-4 fp32 / 3e-3 bf16
forward, 5e-3 gradients; max-norm relative).

Read-after-write: with b = 1 and a unit-norm key, S_t^T k_t = z_t whatever S_{t-1} and the
decay were (the erase removes exactly what the key reads).  Taking q = k makes every output
o_t = w_t * v_t.  One-hot keys are unit-norm exactly in bf16, so this holds for the bf16 path
up to its arithmetic; it is checked at the configurations' full sizes on every forward path
(forward-only records and wide sweep, the segmented sweep, the fused fp32 sweep).  Each output
then depends on its own token's v and w only, so with dS_final = 0 the backward must give
dv = dO * w and dw = dO * v exactly: checked at full size on the one-call backward (segmented
and one-launch state sweeps) and the staged training step."""
import pytest
import torch

import oracle
import linear_attention_sequence_gdn2_amd as gdn2
from linear_attention_sequence_gdn2_amd.inputs import WORKLOADS, make_inputs, make_workload
from _util import oracle_args, rel_err, to_dev

pytestmark = pytest.mark.gpu

FWD_TOL = {"f32": 1e-4, "bf16": 3e-3}
NAMES = ["dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0"]


def _degenerate(inp, case):
    if case == "no_erase":
        inp["b"] = torch.zeros_like(inp["b"])
    elif case == "no_write":
        inp["w"] = torch.zeros_like(inp["w"])
    elif case == "no_decay":
        inp["log_alpha"] = torch.zeros_like(inp["log_alpha"])
    elif case == "full_erase":
        inp["b"] = torch.ones_like(inp["b"])
    else:
        raise ValueError(case)
    return inp


@pytest.mark.parametrize("qkv", ["f32", "bf16"])
@pytest.mark.parametrize("case", ["no_erase", "no_write", "no_decay", "full_erase"])
def test_degenerate_gates_fwd_bwd(case, qkv):
    # ragged T over three chunks, dk != dv, a nonzero start state (so that w = 0 still reads one)
    inp = _degenerate(make_inputs(2, 150, 3, 64, 128, seed=8100, qkv_dtype=qkv, s0_std=0.2, grads=True), case)
    d = to_dev(inp)
    o, sf = gdn2.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"])
    g = gdn2.bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], d["dO"], d["dS_final"])
    torch.cuda.synchronize()
    args = oracle_args(inp)
    o_ref, sf_ref = oracle.fwd(*args)
    ref = oracle.bwd(*args, inp["dO"], inp["dS_final"])
    eo, es = rel_err(o, o_ref), rel_err(sf, sf_ref)
    errs = {n: rel_err(g[n], ref[n]) for n in NAMES}
    print("%s %s: o %.2e S_final %.2e " % (case, qkv, eo, es) + " ".join("%s=%.2e" % kv for kv in errs.items()))
    assert eo < FWD_TOL[qkv] and es < FWD_TOL[qkv], (eo, es)
    bad = {n: e for n, e in errs.items() if not e < 5e-3}
    assert not bad, bad
    if case == "no_write":
        assert float(g["dv"].abs().max()) == 0.0   # dv = dZ * w


def _read_after_write(x, seed):
    """b = 1, q = k = one-hot keys (a random channel per token and head): o_t = w_t * v_t."""
    B, T, H, dk = x["k"].shape
    gen = torch.Generator().manual_seed(seed)
    ch = torch.randint(0, dk, (B, T, H), generator=gen)
    onehot = torch.nn.functional.one_hot(ch, dk).to(x["k"].dtype).contiguous()
    x["q"], x["k"] = onehot, onehot.clone()
    x["b"] = torch.ones_like(x["b"])
    return x


@pytest.mark.parametrize("name,B", [
    ("fwd_bf16_B8H16T2048d128", None),       # forward-only records + wide sweep
    ("long_bf16_B1H16T16384d128", None),     # the segmented sweep (8 segments), nonzero S0
    ("fwdbwd_bf16_B4H16T4096d128", None),    # 64-column tiles on half the CUs, nonzero S0
    ("tiny_f32_B1H2T128d32", 64),            # the fused fp32 sweep, widened to 64 sequences
])
def test_read_after_write_identity_at_full_size(name, B):
    wl = WORKLOADS[name]
    x = _read_after_write(make_workload(wl, **({"B": B} if B else {})), seed=8200)
    d = to_dev(x)
    o, _ = gdn2.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"])
    z = d["w"].float() * d["v"].float()
    torch.cuda.synchronize()
    err = float((o - z).abs().max()) / float(z.abs().max())
    print("%s: max |o - w v| / max |w v| = %.2e" % (name, err))
    assert err < FWD_TOL[wl.qkv_dtype], err


@pytest.mark.parametrize("name,staged", [
    ("fwdbwd_bf16_B4H16T4096d128", False),   # one-call backward (state and reverse sweeps in one launch)
    ("fwd_bf16_B8H16T2048d128", True),       # the staged training step of the bench
    ("long_bf16_B1H16T16384d128", False),    # one-call backward with the segmented state sweep
])
def test_read_after_write_gradients_at_full_size(name, staged):
    """With b = 1 and q = k one-hot, o_t = w_t * v_t depends on no other token, so for
    L = sum(dO * o) (dS_final = 0): dv = dO * w and dw = dO * v exactly."""
    wl = WORKLOADS[name]
    x = _read_after_write(make_workload(wl, grads=True), seed=8300)
    d = to_dev(x)
    if staged:
        factors = gdn2.bwd_factors(d["q"], d["k"], d["log_alpha"], d["b"])
        _, _, states, dstates, _ = gdn2.sweeps(factors, d["v"], d["w"], wl.dk, d["S0"], d["dO"], None)
        g = gdn2.bwd_grads(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["dO"], states, dstates,
                           factors)
    else:
        g = gdn2.bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], d["dO"], None)
    dv_ref = d["dO"] * d["w"]
    dw_ref = d["dO"] * d["v"].float()
    torch.cuda.synchronize()
    ev = float((g["dv"] - dv_ref).abs().max()) / float(dv_ref.abs().max())
    ew = float((g["dw"] - dw_ref).abs().max()) / float(dw_ref.abs().max())
    print("%s: dv %.2e dw %.2e" % (name, ev, ew))
    assert ev < 5e-3 and ew < 5e-3, (ev, ew)
