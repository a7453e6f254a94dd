"""GPU parity of gdn2_chunk_bwd (gate-aware backward) against the fp64 oracle's
reverse recurrence, through the C ABI.

Tolerance: max-norm relative error 5e-3 per gradient tensor (tests/_util.rel_err).
The oracle's own gradients are pinned by finite differences in test_oracle_pins."""
import pytest
import torch

import oracle
import linear_attention_sequence_gdn2_amd as gdn2
from linear_attention_sequence_gdn2_amd.inputs import WORKLOADS, make_inputs, make_workload
from _util import oracle_args, rel_err, sweeps_fuse, to_dev

pytestmark = pytest.mark.gpu

TOL = 5e-3
NAMES = ["dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0"]


def _run(inp, tol=TOL, with_dsf=True):
    d = to_dev(inp)
    dsf = d["dS_final"] if with_dsf else None
    g = gdn2.bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], d["dO"], dsf)
    torch.cuda.synchronize()
    ref = oracle.bwd(*oracle_args(inp), inp["dO"], inp["dS_final"] if with_dsf else None)
    errs = {n: rel_err(g[n], ref[n]) for n in NAMES}
    print(" ".join("%s=%.2e" % kv for kv in errs.items()))
    bad = {n: e for n, e in errs.items() if not e < tol}
    assert not bad, bad


def test_tiny_f32_workload_grads():
    wl = WORKLOADS["tiny_f32_B1H2T128d32"]
    _run(make_workload(wl, grads=True, s0_std=0.02))


@pytest.mark.parametrize("B,T,H,dk,dv,qkv,s0,dsf", [
    (1, 1, 1, 32, 32, "f32", 0.5, True),
    (1, 64, 2, 64, 64, "f32", 0.5, False),
    (2, 65, 1, 128, 128, "f32", 0.5, True),
    (1, 200, 3, 128, 128, "bf16", 0.02, True),
    (2, 333, 2, 64, 128, "bf16", 0.0, True),
    (1, 130, 2, 128, 32, "bf16", 0.1, False),
    (3, 257, 2, 32, 64, "f32", 0.1, True),
])
def test_small_shapes_grads(B, T, H, dk, dv, qkv, s0, dsf):
    inp = make_inputs(B, T, H, dk, dv, seed=7 * B + T + dk + 3 * dv, qkv_dtype=qkv, s0_std=s0, grads=True)
    _run(inp, with_dsf=dsf)


# The reverse sweep's value-tile width follows the number of heads (the widths named below are
# those on 256 CUs): 64 columns when B*H*dv/64 >= CUs, 16 when B*H*dv/16 <= CUs, else 32.
# Ragged T at each width, through the staged entry points (gdn2_chunk_bwd_reverse on its own).
@pytest.mark.parametrize("B,T,H,dk,dv", [
    (8, 100, 16, 128, 128),   # 64 columns
    (3, 130, 16, 128, 128),   # 32
    (1, 300, 16, 128, 128),   # 16
    (2, 129, 16, 64, 128),    # 16, dk 64
])
def test_reverse_tile_widths(B, T, H, dk, dv):
    inp = make_inputs(B, T, H, dk, dv, seed=B * T + H + dk, s0_std=0.05, grads=True)
    d = to_dev(inp)
    factors = gdn2.bwd_factors(d["q"], d["k"], d["log_alpha"], d["b"])
    _, _, states = gdn2.fwd_factored(factors, d["v"], d["w"], dk, d["S0"], want_o=False)
    dstates, dS0 = gdn2.bwd_reverse(factors, d["dO"], dk, d["dS_final"])
    g = gdn2.bwd_grads(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["dO"], states, dstates, factors)
    g["dS0"] = dS0
    torch.cuda.synchronize()
    ref = oracle.bwd(*oracle_args(inp), inp["dO"], inp["dS_final"])
    errs = {n: rel_err(g[n], ref[n]) for n in NAMES}
    print(" ".join("%s=%.2e" % kv for kv in errs.items()))
    bad = {n: e for n, e in errs.items() if not e < TOL}
    assert not bad, bad


# The one-call backward runs its state sweep and the reverse sweep in one launch where both
# sweeps' 64-column tiles fit one workgroup per CU (and the sequence is not segmented): the
# same gradients as the staged entry points, whose states-only sweep takes narrower tiles there.
@pytest.mark.parametrize("B,T,H,dk,dv,extra", [
    (4, 200, 16, 128, 128, {"s0_std": 0.1}),
    (2, 129, 8, 64, 128, {}),
    (2, 150, 4, 128, 128, {"gate_logits": True}),
    (2, 150, 4, 128, 128, {"gates": "gdn", "token_gates": True}),
])
def test_one_call_backward_with_fused_sweeps(B, T, H, dk, dv, extra):
    inp = make_inputs(B, T, H, dk, dv, seed=B * T + H + dk + 1, grads=True, **extra)
    d = to_dev(inp)
    if not sweeps_fuse(B, H, dk, dv):
        pytest.skip("the two sweeps take one launch only with at least 2 B H dv / 64 CUs")
    assert gdn2.sweeps_fused(B, T, H, dk, dv)
    g = gdn2.bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], d["dO"], d["dS_final"])
    factors = gdn2.bwd_factors(d["q"], d["k"], d["log_alpha"], d["b"])
    _, _, states = gdn2.fwd_factored(factors, d["v"], d["w"], dk, d["S0"], want_o=False)
    dstates, dS0 = gdn2.bwd_reverse(factors, d["dO"], dk, d["dS_final"])
    g2 = gdn2.bwd_grads(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["dO"], states, dstates, factors)
    g2["dS0"] = dS0
    torch.cuda.synchronize()
    for n in NAMES:
        assert float((g[n] - g2[n]).abs().max()) <= 1e-3 * float(g2[n].abs().max()), n


def test_full_size_fwdbwd_workload():
    wl = WORKLOADS["fwdbwd_bf16_B4H16T4096d128"]
    _run(make_workload(wl))


@pytest.mark.parametrize("B,T,H,dk,dv,qkv", [
    (1, 64 * 257 - 30, 1, 64, 64, "bf16"),    # 257 chunks: one workgroup walks two items, the rest one
    (2, 64 * 200 + 7, 1, 128, 64, "bf16"),    # 402 chunks: some workgroups two items, ragged tail
    (1, 64 * 255, 1, 32, 64, "f32"),          # 255 chunks: fewer items than workgroups would be
])
def test_chunk_gradient_work_split(B, T, H, dk, dv, qkv):
    """The chunk-gradient kernel is persistent (one workgroup per CU; a workgroup loads its next
    item's record and first value tile during the current item, and its last item loads its own
    again): item counts just above, well above and below the workgroup count, against the
    oracle."""
    _run(make_inputs(B, T, H, dk, dv, seed=9900 + T + dk, qkv_dtype=qkv, s0_std=0.1, grads=True))
