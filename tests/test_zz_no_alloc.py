"""gdn2_chunk_fwd_noalloc (the forward without allocation, records in the library's static
scratch) against gdn2_chunk_fwd (records in a workspace) through the C ABI: two calls in a row,
the second on a smaller input, for the bf16 training shape's layout and for fp32 q/k/v with a
start state.  The same kernels run on the same inputs, so the results must be identical."""
import ctypes

import pytest
import torch

import linear_attention_sequence_gdn2_amd as gdn2
from linear_attention_sequence_gdn2_amd.inputs import make_inputs
from _util import to_dev

pytestmark = pytest.mark.gpu


def _both(B, T, H, dk, dv, seed, **kw):
    inp = make_inputs(B, T, H, dk, dv, seed=seed, **kw)
    d = to_dev(inp)
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"])
    o_ref, sf_ref = gdn2.fwd(*args)
    o, sf = gdn2.fwd_noalloc(*args)
    torch.cuda.synchronize()
    return (o, sf), (o_ref, sf_ref)


@pytest.mark.parametrize("first,second", [
    # batch groups: 2 x (16 heads x 32 chunks) of records fit 256 MiB, so B = 8 runs as 4 groups
    ((8, 2048, 16, 128, 128, {}), (3, 333, 16, 128, 128, {})),
    ((2, 700, 4, 64, 64, {"qkv_dtype": "f32", "s0_std": 0.1}), (1, 65, 2, 64, 64, {"qkv_dtype": "f32"})),
])
def test_noalloc_forward_matches_workspace_forward(first, second):
    for i, (B, T, H, dk, dv, kw) in enumerate((first, second)):
        (o, sf), (o_ref, sf_ref) = _both(B, T, H, dk, dv, seed=9500 + 7 * i + T, **kw)
        assert torch.equal(o, o_ref), ("o", i)
        assert torch.equal(sf, sf_ref), ("S_final", i)


def test_noalloc_rejects_what_does_not_fit():
    lib = gdn2.load()
    assert lib.gdn2_chunk_fwd_noalloc_max_bytes() == 256 << 20
    # one batch element of 16 heads x 16384 tokens needs over 600 MB of records
    s = gdn2.make_shape(1, 16384, 16, 128, 128, torch.bfloat16)
    f = ctypes.c_void_p(0x10000)
    assert lib.gdn2_chunk_fwd_noalloc(ctypes.byref(s), f, f, f, f, f, f, None, f, None, None) == 5
