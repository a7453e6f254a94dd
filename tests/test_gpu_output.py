"""GPU parity of the output epilogue (gdn2_output_fwd / gdn2_output_bwd): RMS norm over
the value channels of each (b, t, h), per-channel weight, output gate.

The reference is the fp64 oracle (oracle.output_fwd / oracle.output_bwd, pinned by
closed forms, invariances and central differences in test_oracle_pins) on the same
inputs.  Tolerances (max-norm relative): a few fp32 operations per element give about
1e-6, so fp32 results are held to 1e-5; dweight sums up to B*T*H rows in fp32 and is
held to 1e-4; a bf16 y carries one rounding to nearest even (relative 2^-9), held to 4e-3."""
import numpy as np
import pytest
import torch

import oracle
import linear_attention_sequence_gdn2_amd as gdn2
from linear_attention_sequence_gdn2_amd.inputs import make_inputs, make_output_inputs
from _util import rel_err, to_dev

pytestmark = pytest.mark.gpu


def _dev(x):
    return {k: v.cuda() for k, v in x.items()}


@pytest.mark.parametrize("B,T,H,dv,g_dtype,y_bf16,use_weight", [
    (1, 1, 1, 32, "f32", False, True),      # a single row
    (1, 7, 3, 64, "f32", False, False),     # 21 rows, less than one workgroup
    (2, 65, 3, 128, "bf16", False, True),   # ragged tail of rows
    (3, 100, 2, 128, "f32", True, True),    # bf16 output
    (2, 333, 4, 32, "bf16", True, False),
    (2, 4500, 8, 64, "f32", False, True),   # more row blocks than the backward grid (1024 workgroups)
])
def test_output_epilogue_small_shapes(B, T, H, dv, g_dtype, y_bf16, use_weight):
    x = make_output_inputs(B, T, H, dv, seed=9000 + T + dv, g_dtype=g_dtype)
    d = _dev(x)
    wt = d["weight"] if use_weight else None
    eps = 1e-6
    y = gdn2.output_fwd(d["o"], d["g"], wt, eps, out_dtype=torch.bfloat16 if y_bf16 else torch.float32)
    gr = gdn2.output_bwd(d["o"], d["g"], wt, eps, d["dy"])
    torch.cuda.synchronize()
    xw = x["weight"] if use_weight else None
    y_ref = oracle.output_fwd(x["o"], x["g"], xw, eps)
    ref = oracle.output_bwd(x["o"], x["g"], xw, eps, x["dy"])
    ey = rel_err(y, y_ref)
    errs = {n: rel_err(gr[k], ref[n]) for k, n in (("dO", "do"), ("dg", "dg"), ("dweight", "dweight"))}
    print("epilogue y %.2e " % ey + " ".join("%s=%.2e" % kv for kv in errs.items()))
    assert ey < (4e-3 if y_bf16 else 1e-5)
    assert errs["do"] < 1e-5 and errs["dg"] < 1e-5 and errs["dweight"] < 1e-4, errs


def test_output_epilogue_training_shape_and_reproducible():
    """B8 T2048 H16 dv128 (the training shape): parity and bitwise-equal repeats."""
    x = make_output_inputs(8, 2048, 16, 128, seed=9100, g_dtype="bf16")
    d = _dev(x)
    y = gdn2.output_fwd(d["o"], d["g"], d["weight"], 1e-6, out_dtype=torch.bfloat16)
    g1 = gdn2.output_bwd(d["o"], d["g"], d["weight"], 1e-6, d["dy"])
    g2 = gdn2.output_bwd(d["o"], d["g"], d["weight"], 1e-6, d["dy"])
    torch.cuda.synchronize()
    for k in ("dO", "dg", "dweight"):
        assert torch.equal(g1[k], g2[k]), k
    assert rel_err(y, oracle.output_fwd(x["o"], x["g"], x["weight"], 1e-6)) < 4e-3
    ref = oracle.output_bwd(x["o"], x["g"], x["weight"], 1e-6, x["dy"])
    e = {k: rel_err(g1[k], ref[n]) for k, n in (("dO", "do"), ("dg", "dg"), ("dweight", "dweight"))}
    print("training-shape epilogue", e)
    assert e["dO"] < 1e-5 and e["dg"] < 1e-5 and e["dweight"] < 1e-4, e


def test_output_epilogue_degenerate_rows():
    """A zero row gives y = 0 and finite gradients when eps > 0; eps = 0 is exact RMS."""
    x = make_output_inputs(1, 40, 2, 64, seed=9200)
    x["o"][0, 3, 1] = 0.0
    d = _dev(x)
    y = gdn2.output_fwd(d["o"], d["g"], d["weight"], 1e-5)
    gr = gdn2.output_bwd(d["o"], d["g"], d["weight"], 1e-5, d["dy"])
    y0 = gdn2.output_fwd(d["o"][:, :3].contiguous(), torch.ones_like(d["g"][:, :3]), None, 0.0)
    torch.cuda.synchronize()
    assert torch.all(y[0, 3, 1] == 0) and torch.all(torch.isfinite(gr["dO"]))
    assert rel_err(gr["dO"], oracle.output_bwd(x["o"], x["g"], x["weight"], 1e-5, x["dy"])["do"]) < 1e-5
    ms = (y0.double() ** 2).mean(-1).cpu().numpy()
    assert np.allclose(ms, 1.0, rtol=0, atol=1e-5)


def test_operator_with_epilogue_chain():
    """Operator forward then epilogue; epilogue backward feeds the operator backward:
    against the oracle chain on the same inputs."""
    inp = make_inputs(2, 130, 2, 64, 128, seed=9300, s0_std=0.1, grads=True)
    ex = make_output_inputs(2, 130, 2, 128, seed=9301, g_dtype="bf16")
    d, de = to_dev(inp), _dev(ex)
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    o, sf, states = gdn2.fwd_states(*args, d["S0"])
    y = gdn2.output_fwd(o, de["g"], de["weight"], 1e-6)
    ge = gdn2.output_bwd(o, de["g"], de["weight"], 1e-6, de["dy"])
    g = gdn2.bwd_saved(*args, states, ge["dO"], None)
    torch.cuda.synchronize()
    oa = [inp["q32"], inp["k32"], inp["v32"], inp["log_alpha"], inp["b"], inp["w"], inp["S0"]]
    o_ref, _ = oracle.fwd(*oa)
    y_ref = oracle.output_fwd(o_ref, ex["g"], ex["weight"], 1e-6)
    ge_ref = oracle.output_bwd(o_ref, ex["g"], ex["weight"], 1e-6, ex["dy"])
    g_ref = oracle.bwd(*oa, ge_ref["do"], None)
    errs = {"y": rel_err(y, y_ref), "dg": rel_err(ge["dg"], ge_ref["dg"]),
            "dweight": rel_err(ge["dweight"], ge_ref["dweight"])}
    errs.update({n: rel_err(g[n], g_ref[n]) for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0")})
    print(" ".join("%s=%.2e" % kv for kv in errs.items()))
    assert errs["y"] < 3e-3 and errs["dg"] < 3e-3 and errs["dweight"] < 3e-3, errs
    bad = {n: e for n, e in errs.items() if not e < 5e-3}
    assert not bad, bad
