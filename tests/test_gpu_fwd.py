"""GPU parity of gdn2_chunk_fwd against the fp64 oracle, through the C ABI.

Tolerances (max-norm relative error, see tests/_util.rel_err): 1e-4 for fp32
q/k/v, 3e-3 for bf16 q/k/v (the oracle reads the same bf16-rounded values)."""
import pytest
import torch

import oracle
import linear_attention_sequence_gdn2_amd as gdn2
from linear_attention_sequence_gdn2_amd.inputs import WORKLOADS, make_inputs, make_workload
from _util import oracle_args, rel_err, to_dev

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 3e-3}


def _run(inp, qkv):
    d = to_dev(inp)
    o, sf = gdn2.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"])
    torch.cuda.synchronize()
    o_ref, sf_ref = oracle.fwd(*oracle_args(inp))
    eo, es = rel_err(o, o_ref), rel_err(sf, sf_ref)
    print("o err %.3e  S_final err %.3e" % (eo, es))
    assert eo < TOL[qkv] and es < TOL[qkv], (eo, es)


def test_tiny_f32_workload():
    wl = WORKLOADS["tiny_f32_B1H2T128d32"]
    _run(make_workload(wl), "f32")


@pytest.mark.parametrize("B,T,H,dk,dv,qkv,s0", [
    (1, 1, 1, 32, 32, "f32", 0.5),        # a single token
    (1, 64, 2, 64, 64, "f32", 0.5),       # exactly one chunk
    (2, 65, 1, 128, 128, "f32", 0.5),     # one token into the second chunk
    (1, 200, 3, 128, 128, "bf16", 0.02),  # ragged tail, value tiles
    (2, 333, 2, 64, 128, "bf16", 0.0),    # dk != dv
    (1, 130, 2, 128, 32, "bf16", 0.1),
    (3, 257, 2, 32, 64, "f32", 0.1),
])
def test_small_shapes(B, T, H, dk, dv, qkv, s0):
    inp = make_inputs(B, T, H, dk, dv, seed=B * 1000 + T + dk + dv, qkv_dtype=qkv, s0_std=s0)
    _run(inp, qkv)


@pytest.mark.parametrize("name", ["fwd_bf16_B8H16T2048d128", "long_bf16_B1H16T16384d128",
                                  "kda_bf16_B4H16T4096d128", "gdn_bf16_B4H16T4096d128"])
def test_full_size_workloads(name):
    wl = WORKLOADS[name]
    _run(make_workload(wl), wl.qkv_dtype)
