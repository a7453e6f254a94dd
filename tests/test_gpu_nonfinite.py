"""Non-finite inputs propagate and stay where the rule puts them.

A NaN or an infinity in one head's inputs reaches that head's outputs (the recurrence carries
it from its chunk on), and no other head's: (batch, head) pairs are independent, so every other
head's outputs and gradients must equal those of the clean inputs bit for bit.  The kernels have
no data-dependent loop or wait, so such inputs end like any other call.  Checked for a NaN key,
an infinite value, a NaN decay and a NaN erase gate, forward and one-call backward, on the wide
sweep (bf16) and the fp32 sweep."""
import pytest
import torch

import linear_attention_sequence_gdn2_amd as gdn2
from linear_attention_sequence_gdn2_amd.inputs import make_inputs
from _util import to_dev

pytestmark = pytest.mark.gpu

B, T, H = 2, 200, 3
BAD_B, BAD_T, BAD_H = 1, 70, 1        # token 70: the second chunk (tokens 64 .. 127)


@pytest.mark.parametrize("qkv", ["bf16", "f32"])
@pytest.mark.parametrize("where,value", [("k", float("nan")), ("v", float("inf")), ("log_alpha", float("nan")),
                                         ("b", float("nan"))])
def test_nonfinite_input_stays_in_its_head(qkv, where, value):
    inp = make_inputs(B, T, H, 128, 128, seed=9600, qkv_dtype=qkv, s0_std=0.1, grads=True)
    d = to_dev(inp)
    bad = dict(d)
    bad[where] = d[where].clone()
    bad[where][BAD_B, BAD_T, BAD_H, 5] = value
    print("case", qkv, where, value, flush=True)
    outs = []
    for x in (d, bad):
        args = (x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], x["S0"])
        o, sf = gdn2.fwd(*args)
        g = gdn2.bwd(*args, x["dO"], x["dS_final"])
        outs.append((o, sf, g))
    torch.cuda.synchronize()
    (o0, sf0, g0), (o1, sf1, g1) = outs
    heads = [(b, h) for b in range(B) for h in range(H) if (b, h) != (BAD_B, BAD_H)]
    for b, h in heads:
        assert torch.equal(o0[b, :, h], o1[b, :, h]), (b, h)
        assert torch.equal(sf0[b, h], sf1[b, h]), (b, h)
        for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw"):
            assert torch.equal(g0[n][b, :, h], g1[n][b, :, h]), (n, b, h)
        assert torch.equal(g0["dS0"][b, h], g1["dS0"][b, h]), (b, h)
    # the poisoned head: clean before the poisoned chunk, non-finite from it on
    o = o1[BAD_B, :, BAD_H]
    assert torch.equal(o[:64], o0[BAD_B, :64, BAD_H])
    assert not bool(torch.isfinite(o[64:]).all())
    assert not bool(torch.isfinite(sf1[BAD_B, BAD_H]).all())
    assert any(not bool(torch.isfinite(g1[n][BAD_B, :, BAD_H]).all())
               for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw"))
    if where == "v":
        # the start state's gradient depends on the key side and dO only, not on v
        assert torch.equal(g1["dS0"][BAD_B, BAD_H], g0["dS0"][BAD_B, BAD_H])
    else:
        assert not bool(torch.isfinite(g1["dS0"][BAD_B, BAD_H]).all())
