"""GPU invariants of the operator (through the C ABI): the staged entry points
agree with the one-call forms, sequences can be split across calls, results are
bitwise reproducible, every output element is written, and permuting value
channels permutes the outputs."""
import pytest
import torch

import linear_attention_sequence_gdn2_amd as gdn2
from linear_attention_sequence_gdn2_amd.inputs import make_inputs
from _util import to_dev

pytestmark = pytest.mark.gpu


def _dev(B=2, T=300, H=2, dk=128, dv=128, seed=11, qkv="bf16", s0=0.02):
    return to_dev(make_inputs(B, T, H, dk, dv, seed=seed, qkv_dtype=qkv, s0_std=s0, grads=True))


def _fargs(d):
    return (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"])


def test_staged_forward_and_backward_match_one_call_forms():
    d = _dev()
    o1, s1 = gdn2.fwd(*_fargs(d))
    o2, s2, states = gdn2.fwd_states(*_fargs(d))
    st2 = gdn2.chunk_states(d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"])
    # the backward chain: factors, the states-only sweep from them (what the one-call backward
    # recomputes), reverse sweep, token gradients
    factors = gdn2.bwd_factors(d["q"], d["k"], d["log_alpha"], d["b"])
    _, _, st_s = gdn2.fwd_factored(factors, d["v"], d["w"], 128, d["S0"], want_o=False)
    dstates, dS0 = gdn2.bwd_reverse(factors, d["dO"], 128, d["dS_final"])
    g2 = gdn2.bwd_grads(*_fargs(d)[:6], d["dO"], st_s, dstates, factors)
    g2["dS0"] = dS0
    g1 = gdn2.bwd(*_fargs(d), d["dO"], d["dS_final"])
    g4 = gdn2.bwd_saved(*_fargs(d)[:6], st_s, d["dO"], d["dS_final"])
    # the training forward from the factors (o and states)
    o3, s3, st3 = gdn2.fwd_factored(factors, d["v"], d["w"], 128, d["S0"])
    torch.cuda.synchronize()
    # fwd_states sweeps o and the states, chunk_states the states alone (a narrower kernel where
    # there are few heads): equal up to rounding
    assert float((states - st2).abs().max()) <= 1e-3 * float(st2.abs().max())
    # the one-call backward is exactly this chain (same kernels, same inputs)
    for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0"):
        assert torch.equal(g1[n], g2[n]), n
        assert torch.equal(g4[n], g2[n]), n
    # the inference forward (forward-only records), the o + states sweep and the states-only
    # sweep (which takes narrower tiles when there are few heads): equal up to rounding
    for x, y in ((o1, o2), (s1, s2), (o1, o3), (s1, s3), (states, st3), (st_s, st3)):
        assert float((x - y).abs().max()) <= 1e-3 * float(y.abs().max())
    # states[0] is the start state
    for st in (states, st3, st_s):
        assert torch.equal(st[:, :, 0], d["S0"])


def test_split_sequence_chains_through_the_state():
    d = _dev(T=320, qkv="f32", s0=0.3)
    o, sf = gdn2.fwd(*_fargs(d))
    c = 128  # a chunk boundary, so both halves use the same chunking
    p1 = [t[:, :c].contiguous() for t in _fargs(d)[:6]]
    p2 = [t[:, c:].contiguous() for t in _fargs(d)[:6]]
    o1, s1 = gdn2.fwd(*p1, d["S0"])
    o2, s2 = gdn2.fwd(*p2, s1)
    torch.cuda.synchronize()
    err_o = (torch.cat([o1, o2], 1) - o).abs().max() / o.abs().max()
    err_s = (s2 - sf).abs().max() / sf.abs().max()
    assert err_o < 1e-5 and err_s < 1e-5, (err_o, err_s)


def test_results_are_bitwise_reproducible():
    d = _dev(B=3, T=257, seed=5)
    runs = [gdn2.fwd(*_fargs(d)) for _ in range(3)]
    grads = [gdn2.bwd(*_fargs(d), d["dO"], d["dS_final"]) for _ in range(2)]
    torch.cuda.synchronize()
    for o, s in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(s, runs[0][1])
    for n in grads[0]:
        assert torch.equal(grads[0][n], grads[1][n]), n


def test_every_output_element_is_written():
    d = _dev(B=1, T=130, H=3, dk=64, dv=128, seed=9)
    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    nc = (T + 63) // 64
    states = torch.full((B, H, nc, dk, dv), float("nan"), device="cuda")
    o, sf, states = gdn2.fwd_states(*_fargs(d), states=states)
    dstates = torch.full_like(states, float("nan"))
    factors = gdn2.bwd_factors(d["q"], d["k"], d["log_alpha"], d["b"])
    dstates, dS0 = gdn2.bwd_reverse(factors, d["dO"], dk, d["dS_final"], dstates=dstates)
    g = gdn2.bwd_grads(*_fargs(d)[:6], d["dO"], states, dstates, factors)
    torch.cuda.synchronize()
    for t in [o, sf, states, dstates, dS0] + list(g.values()):
        assert torch.isfinite(t).all()


def test_value_channel_permutation_equivariance():
    d = _dev(B=1, T=200, H=2, seed=21, qkv="f32")
    perm = torch.randperm(d["v"].shape[-1], generator=torch.Generator().manual_seed(0)).cuda()
    o, sf = gdn2.fwd(*_fargs(d))
    o2, sf2 = gdn2.fwd(d["q"], d["k"], d["v"][..., perm].contiguous(), d["log_alpha"], d["b"],
                       d["w"][..., perm].contiguous(), d["S0"][..., perm].contiguous())
    torch.cuda.synchronize()
    assert (o2 - o[..., perm]).abs().max() <= 1e-5 * o.abs().max()
    assert (sf2 - sf[..., perm]).abs().max() <= 1e-5 * sf.abs().max()


def test_argument_errors_surface_as_exceptions():
    d = _dev(B=1, T=64, H=1)
    with pytest.raises(ValueError):
        gdn2.fwd(d["q"], d["k"], d["v"], d["log_alpha"][..., :64].contiguous(), d["b"], d["w"])
    with pytest.raises(ValueError):
        gdn2.fwd(d["q"], d["k"].transpose(1, 2), d["v"], d["log_alpha"], d["b"], d["w"])


def test_every_output_is_written_over_poisoned_memory(monkeypatch):
    """Every tensor the binding allocates (outputs, workspaces, factor buffers) starts out as
    NaN (bytes as 0xFF); every output of every entry point must come back finite: the kernels
    write all of it and read nothing they have not written."""
    real_empty = torch.empty

    def poisoned_empty(*shape, **kw):
        t = real_empty(*shape, **kw)
        if t.is_floating_point():
            t.fill_(float("nan"))
        else:
            t.fill_(255)
        return t

    monkeypatch.setattr(torch, "empty", poisoned_empty)
    for qkv, dv in (("bf16", 128), ("f32", 64), ("bf16", 32)):   # wide sweep, fp32 sweep, narrow tiles
        d = _dev(B=2, T=150, H=3, dk=128, dv=dv, seed=31, qkv=qkv)
        outs = list(gdn2.fwd(*_fargs(d)))
        outs += list(gdn2.fwd_states(*_fargs(d)))
        g = gdn2.bwd(*_fargs(d), d["dO"], d["dS_final"])
        outs += list(g.values())
        factors = gdn2.bwd_factors(d["q"], d["k"], d["log_alpha"], d["b"])
        o, sf, states = gdn2.fwd_factored(factors, d["v"], d["w"], 128, d["S0"])
        _, _, st_s = gdn2.fwd_factored(factors, d["v"], d["w"], 128, d["S0"], want_o=False)
        dstates, dS0 = gdn2.bwd_reverse(factors, d["dO"], 128, d["dS_final"])
        outs += [o, sf, states, st_s, dstates, dS0]
        outs += list(gdn2.bwd_grads(*_fargs(d)[:6], d["dO"], states, dstates, factors).values())
        torch.cuda.synchronize()
        for t in outs:
            assert t is not None and bool(torch.isfinite(t).all()), qkv
