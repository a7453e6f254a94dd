"""GPU parity of the forward sweep from the factor buffer (gdn2_chunk_fwd_factored).

The adjoint-factor kernel (gdn2_chunk_bwd_factors) writes the key-side operands of
every chunk; the sweep takes them from there and reads only v, w and S0.  Outputs
are checked against the fp64 oracle at the forward's tolerances (1e-4 fp32 q/k/v,
3e-3 bf16; max-norm relative), states against the oracle's state after every chunk,
and the whole training chain (factors, this forward, reverse sweep, token gradients)
against the oracle's gradients (5e-3)."""
import numpy as np
import pytest
import torch

import oracle
import linear_attention_sequence_gdn2_amd as gdn2
from linear_attention_sequence_gdn2_amd.inputs import WORKLOADS, make_inputs, make_workload
from _util import device_cus, oracle_args, rel_err, sweeps_fuse, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 3e-3}
NAMES = ["dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0"]


def _oracle_inputs(inp):
    if inp.get("gate_logits"):
        return [inp["q32"], inp["k32"], inp["v32"], *oracle.gates_from_logits(inp["log_alpha"], inp["b"], inp["w"]),
                inp["S0"]]
    if inp.get("gate_scalar"):
        dk, dv = inp["q"].shape[-1], inp["v"].shape[-1]
        return [inp["q32"], inp["k32"], inp["v32"],
                *oracle.gates_per_token(inp["log_alpha"], inp["b"], inp["w"], dk, dv, inp["gate_scalar"]), inp["S0"]]
    return oracle_args(inp)


def _oracle_states(args, T):
    """States before every chunk: the oracle chained over the input one chunk at a time."""
    q, k, v, la, b, w, S0 = [oracle._f64(x) if x is not None else None for x in args]
    B, _, H, dk = q.shape
    dv = v.shape[-1]
    out = []
    S = S0
    for c0 in range(0, T, 64):
        out.append(np.zeros((B, H, dk, dv)) if S is None else S)
        sl = slice(c0, min(c0 + 64, T))
        _, S = oracle.fwd(q[:, sl], k[:, sl], v[:, sl], la[:, sl], b[:, sl], w[:, sl], S)
    return np.stack(out, axis=2)


def _run(inp, tol, check_states=False):
    d = to_dev(inp)
    dk = d["q"].shape[-1]
    T = d["q"].shape[1]
    factors = gdn2.bwd_factors(d["q"], d["k"], d["log_alpha"], d["b"])
    o, sf, states = gdn2.fwd_factored(factors, d["v"], d["w"], dk, d["S0"])
    torch.cuda.synchronize()
    args = _oracle_inputs(inp)
    o_ref, sf_ref = oracle.fwd(*args)
    eo, es = rel_err(o, o_ref), rel_err(sf, sf_ref)
    print("factored forward: o err %.3e  S_final err %.3e" % (eo, es))
    assert eo < tol and es < tol, (eo, es)
    if check_states:
        et = rel_err(states, _oracle_states(args, T))
        print("states err %.3e" % et)
        assert et < tol
    return d, factors, states


@pytest.mark.parametrize("B,T,H,dk,dv,qkv,s0", [
    (1, 1, 1, 32, 32, "f32", 0.5),
    (1, 64, 2, 64, 64, "f32", 0.5),
    (2, 65, 1, 128, 128, "f32", 0.5),
    (1, 200, 3, 128, 128, "bf16", 0.02),
    (2, 333, 2, 64, 128, "bf16", 0.0),
    (1, 130, 2, 128, 32, "bf16", 0.1),
    (3, 257, 2, 32, 64, "f32", 0.1),
])
def test_factored_forward_small_shapes(B, T, H, dk, dv, qkv, s0):
    inp = make_inputs(B, T, H, dk, dv, seed=11 * B + T + dk + dv, qkv_dtype=qkv, s0_std=s0)
    _run(inp, TOL[qkv], check_states=True)


def test_factored_forward_modes_agree():
    """o only and o + states: the same values (one kernel).  With few heads the states-only
    sweep takes narrower tiles in another kernel: equal up to rounding there (the wide-tile
    test below checks it bit for bit where both take the same kernel)."""
    inp = make_inputs(2, 150, 2, 128, 64, seed=4711, s0_std=0.1)
    d = to_dev(inp)
    factors = gdn2.bwd_factors(d["q"], d["k"], d["log_alpha"], d["b"])
    o1, s1, st1 = gdn2.fwd_factored(factors, d["v"], d["w"], 128, d["S0"])
    o2, s2, _ = gdn2.fwd_factored(factors, d["v"], d["w"], 128, d["S0"], want_states=False)
    _, s3, st3 = gdn2.fwd_factored(factors, d["v"], d["w"], 128, d["S0"], want_o=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    for x, y in ((s3, s1), (st3, st1)):
        assert float((x - y).abs().max()) <= 1e-3 * float(y.abs().max())


@pytest.mark.parametrize("name", ["fwd_bf16_B8H16T2048d128", "long_bf16_B1H16T16384d128",
                                  "kda_bf16_B4H16T4096d128"])
def test_factored_forward_full_size(name):
    wl = WORKLOADS[name]
    _run(make_workload(wl), TOL[wl.qkv_dtype])


@pytest.mark.parametrize("variant", ["logits", "token_gates"])
def test_factored_forward_gate_formats(variant):
    if variant == "logits":
        inp = make_inputs(2, 130, 2, 128, 128, seed=4712, s0_std=0.1, gate_logits=True)
    else:
        inp = make_inputs(2, 130, 2, 128, 128, seed=4713, s0_std=0.1, gates="gdn", token_gates=True)
    _run(inp, TOL["bf16"], check_states=True)


def test_training_chain_from_factors():
    """factors -> factored forward (o, states) -> reverse sweep -> token gradients, on the
    B4 T4096 H16 d128 training workload, against the oracle's forward and gradients."""
    inp = make_workload(WORKLOADS["fwdbwd_bf16_B4H16T4096d128"])
    d, factors, states = _run(inp, TOL["bf16"])
    dstates, dS0 = gdn2.bwd_reverse(factors, d["dO"], 128, d["dS_final"])
    g = gdn2.bwd_grads(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["dO"], states, dstates, factors)
    g["dS0"] = dS0
    torch.cuda.synchronize()
    ref = oracle.bwd(*_oracle_inputs(inp), inp["dO"], inp["dS_final"])
    errs = {n: rel_err(g[n], ref[n]) for n in NAMES}
    print(" ".join("%s=%.2e" % kv for kv in errs.items()))
    bad = {n: e for n, e in errs.items() if not e < 5e-3}
    assert not bad, bad


# Shapes with at least one 64-column value tile per CU take the eight-wave sweep in every mode
# (B*H*dv/64 >= 256); ragged T, both key widths it covers, every gate format and mode.
@pytest.mark.parametrize("B,T,H,dk,dv,extra", [
    (8, 33, 16, 128, 128, {"s0_std": 0.2}),     # one partial chunk
    (8, 64, 16, 128, 128, {}),                  # exactly one chunk
    (8, 200, 16, 128, 128, {}),
    (4, 130, 32, 64, 128, {}),
    (2, 65, 64, 128, 128, {"s0_std": 0.1}),
    (8, 150, 16, 128, 128, {"gate_logits": True}),
    (8, 150, 16, 128, 128, {"gates": "gdn", "token_gates": True}),
    (8, 150, 16, 128, 128, {"gates": "erase_mean", "token_gates": True}),
])
def test_factored_forward_wide_tiles(B, T, H, dk, dv, extra):
    inp = make_inputs(B, T, H, dk, dv, seed=B + T + H + dk, **extra)
    d, factors, states = _run(inp, TOL["bf16"], check_states=True)
    # states-only mode writes the same states
    _, _, st2 = gdn2.fwd_factored(factors, d["v"], d["w"], dk, d["S0"], want_o=False)
    # the inference forward takes forward-only records at these shapes: the same arithmetic
    o_f, sf_f, _ = gdn2.fwd_factored(factors, d["v"], d["w"], dk, d["S0"], want_states=False)
    o_i, sf_i = gdn2.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"])
    torch.cuda.synchronize()
    if B * H * (dv // 64) >= device_cus():
        assert torch.equal(states, st2)
    else:   # the states-only sweep takes the four-wave kernel below full occupancy
        assert float((states - st2).abs().max()) <= 1e-3 * float(st2.abs().max())
    assert torch.equal(o_i, o_f) and torch.equal(sf_i, sf_f)


# With at most half the CUs given a 64-column tile (B*H*dv/64 <= 128), the eight-wave sweep takes
# 32-column tiles: ragged T, both key widths, every gate format, against the oracle (outputs and
# every chunk state) and the inference forward against the factored one bit for bit.
@pytest.mark.parametrize("B,T,H,dk,dv,extra", [
    (4, 150, 16, 128, 128, {"s0_std": 0.2}),
    (2, 65, 16, 64, 128, {}),
    (1, 64, 8, 128, 64, {"s0_std": 0.1}),
    (4, 150, 16, 128, 128, {"gate_logits": True}),
    (4, 150, 16, 128, 128, {"gates": "gdn", "token_gates": True}),
])
def test_factored_forward_32_column_tiles(B, T, H, dk, dv, extra):
    if 2 * B * H * (dv // 64) > device_cus():
        pytest.skip("32-column tiles are taken at most at half the CUs of this device")
    test_factored_forward_wide_tiles(B, T, H, dk, dv, extra)


# gdn2_chunk_sweeps: both sweeps of the training step from one factor buffer; one launch where
# their 64-column tiles together take at most one workgroup per CU (256 CUs), two otherwise.  The
# same bodies run as in the two separate entry points, so the results are the same bit for bit.
@pytest.mark.parametrize("B,T,H,dk,dv,extra,one", [
    (4, 130, 16, 128, 128, {"s0_std": 0.1}, True),      # 256 workgroups: one launch
    (2, 1, 8, 128, 128, {"s0_std": 0.1}, True),         # T = 1
    (1, 64, 4, 64, 64, {"s0_std": 0.1}, True),          # exactly one chunk, dk = dv = 64
    (2, 200, 8, 64, 128, {}, True),                      # dk = 64
    (1, 64 * 20 + 3, 2, 128, 64, {"s0_std": 0.2}, True),
    (2, 150, 4, 128, 128, {"gate_logits": True}, True),
    (2, 150, 4, 128, 128, {"gates": "gdn", "token_gates": True}, True),
    (8, 100, 16, 128, 128, {}, False),                   # 512 workgroups: two launches
    (2, 70, 2, 128, 128, {"qkv_dtype": "f32"}, False),   # fp32 q/k/v: two launches
])
def test_sweeps_entry_matches_separate_calls(B, T, H, dk, dv, extra, one):
    inp = make_inputs(B, T, H, dk, dv, seed=B * 31 + T + H + dk, grads=True, **extra)
    d = to_dev(inp)
    assert one == sweeps_fuse(B, H, dk, dv, inp["q"].dtype == torch.bfloat16) or device_cus() != 256
    assert gdn2.sweeps_fused(B, T, H, dk, dv, d["q"].dtype) == sweeps_fuse(B, H, dk, dv, inp["q"].dtype == torch.bfloat16)
    factors = gdn2.bwd_factors(d["q"], d["k"], d["log_alpha"], d["b"])
    o, sf, st, dst, dS0 = gdn2.sweeps(factors, d["v"], d["w"], dk, d["S0"], d["dO"], d["dS_final"])
    o2, sf2, st2 = gdn2.fwd_factored(factors, d["v"], d["w"], dk, d["S0"])
    dst2, dS02 = gdn2.bwd_reverse(factors, d["dO"], dk, d["dS_final"])
    torch.cuda.synchronize()
    for x, y in ((o, o2), (sf, sf2), (st, st2), (dst, dst2), (dS0, dS02)):
        assert torch.equal(x, y)


def test_training_chain_through_fused_sweeps():
    """factors -> both sweeps in one launch -> token gradients, on a shape the one launch takes,
    against the oracle's forward and gradients."""
    inp = make_inputs(4, 333, 16, 128, 128, seed=4714, s0_std=0.05, grads=True)
    d = to_dev(inp)
    assert gdn2.sweeps_fused(4, 333, 16, 128, 128) == sweeps_fuse(4, 16, 128, 128)
    factors = gdn2.bwd_factors(d["q"], d["k"], d["log_alpha"], d["b"])
    o, sf, states, dstates, dS0 = gdn2.sweeps(factors, d["v"], d["w"], 128, d["S0"], d["dO"], d["dS_final"])
    g = gdn2.bwd_grads(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["dO"], states, dstates, factors)
    g["dS0"] = dS0
    torch.cuda.synchronize()
    o_ref, sf_ref = oracle.fwd(*oracle_args(inp))
    assert rel_err(o, o_ref) < TOL["bf16"] and rel_err(sf, sf_ref) < TOL["bf16"]
    ref = oracle.bwd(*oracle_args(inp), inp["dO"], inp["dS_final"])
    errs = {n: rel_err(g[n], ref[n]) for n in NAMES}
    print(" ".join("%s=%.2e" % kv for kv in errs.items()))
    bad = {n: e for n, e in errs.items() if not e < 5e-3}
    assert not bad, bad


@pytest.mark.parametrize("with_s0,with_dsf,want_state,want_dS0", [
    (False, False, False, False),
    (True, False, True, False),
    (False, True, False, True),
])
def test_sweeps_entry_optional_arguments(with_s0, with_dsf, want_state, want_dS0):
    """The one launch with S0 / dS_final absent (zeros) and S_final / dS0 not wanted."""
    B, T, H, dk, dv = 2, 140, 8, 128, 128
    inp = make_inputs(B, T, H, dk, dv, seed=4715, s0_std=0.1, grads=True)
    d = to_dev(inp)
    assert gdn2.sweeps_fused(B, T, H, dk, dv) == sweeps_fuse(B, H, dk, dv)
    S0 = d["S0"] if with_s0 else None
    dsf = d["dS_final"] if with_dsf else None
    factors = gdn2.bwd_factors(d["q"], d["k"], d["log_alpha"], d["b"])
    o, sf, st, dst, dS0 = gdn2.sweeps(factors, d["v"], d["w"], dk, S0, d["dO"], dsf, want_state=want_state,
                                      want_dS0=want_dS0)
    o2, sf2, st2 = gdn2.fwd_factored(factors, d["v"], d["w"], dk, S0)
    dst2, dS02 = gdn2.bwd_reverse(factors, d["dO"], dk, dsf)
    torch.cuda.synchronize()
    assert (sf is None) != want_state and (dS0 is None) != want_dS0
    assert torch.equal(o, o2) and torch.equal(st, st2) and torch.equal(dst, dst2)
    if want_state:
        assert torch.equal(sf, sf2)
    if want_dS0:
        assert torch.equal(dS0, dS02)
