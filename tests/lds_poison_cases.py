"""Runs every kernel of the library on small seeded cases and saves all results to one file
(argv[1]).  tests/test_gpu_lds_poison.py runs it once with the normal build and once with the
LDS poison-fill build (GDN2_LIBRARY=libgdn2_poison.so) and compares the two files bit for bit.
Each case prints its name before it runs."""
import os
import sys

import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import linear_attention_sequence_gdn2_amd as gdn2  # noqa: E402
from linear_attention_sequence_gdn2_amd.inputs import make_inputs, make_output_inputs  # noqa: E402

# (name, B, T, H, dk, dv, recipe): together they take every launch path of the library
CASES = [
    ("wide_bf16", 2, 150, 40, 128, 128, {"s0_std": 0.1}),          # records + 64-column sweeps, two launches
    ("tile32_bf16", 1, 300, 4, 128, 128, {"s0_std": 0.1}),         # 32-column tiles, sweeps in one launch
    ("narrow_f32", 1, 130, 2, 64, 64, {"qkv_dtype": "f32", "s0_std": 0.1}),   # the four-wave sweep
    ("segmented", 1, 64 * 64 + 5, 2, 64, 64, {"s0_std": 0.1}),    # segmented forward and state sweep
    ("strong_decay", 2, 150, 3, 64, 128, {"decay": "const2", "s0_std": 0.1}),   # exact passes
    ("logits", 2, 150, 3, 128, 128, {"gate_logits": True}),
    ("token_gates", 2, 150, 3, 64, 128, {"gates": "gdn", "token_gates": True}),
]


def main(path):
    dev = torch.device("cuda:0")
    res = {}

    def keep(prefix, **ts):
        for n, t in ts.items():
            if t is not None:
                res["%s.%s" % (prefix, n)] = t.detach().cpu()

    for name, B, T, H, dk, dv, kw in CASES:
        print("case", name, flush=True)
        x = make_inputs(B, T, H, dk, dv, seed=9600 + T + H, grads=True, **kw)
        d = {n: (x[n].to(dev) if x.get(n) is not None else None)
             for n in ("q", "k", "v", "log_alpha", "b", "w", "S0", "dO", "dS_final")}
        args = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"])
        o, sf = gdn2.fwd(*args)
        keep(name + ".fwd", o=o, S_final=sf)
        g = gdn2.bwd(*args, d["dO"], d["dS_final"])
        keep(name + ".bwd", **g)
        factors = gdn2.bwd_factors(d["q"], d["k"], d["log_alpha"], d["b"])
        o2, sf2, states, dstates, dS0 = gdn2.sweeps(factors, d["v"], d["w"], dk, d["S0"], d["dO"], d["dS_final"])
        g2 = gdn2.bwd_grads(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["dO"], states, dstates,
                            factors)
        keep(name + ".staged", o=o2, S_final=sf2, states=states, dstates=dstates, dS0=dS0, **g2)
        torch.cuda.synchronize()

    # the fused epilogue on a shape with one workgroup per head (dv = 64 on 64-column tiles): the
    # shapes whose heads span several workgroups take a cooperative launch, which the runtime can
    # refuse while the test process that starts this one holds the device's cooperative resources
    print("case output epilogue", flush=True)
    x = make_inputs(3, 70, 50, 128, 64, seed=9650, s0_std=0.05)
    ex = make_output_inputs(3, 70, 50, 64, seed=9651, g_dtype="bf16")
    d = {n: (x[n].to(dev) if x.get(n) is not None else None) for n in ("q", "k", "v", "log_alpha", "b", "w", "S0")}
    g, wt, dy = ex["g"].to(dev), ex["weight"].to(dev), ex["dy"].to(dev)
    assert gdn2.fwd_output_fused(3, 70, 50, 128, 64, torch.bfloat16), "the shape should take the fused sweep"
    y, sf, _ = gdn2.fwd_output(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], g, wt, 1e-6, d["S0"],
                               out_dtype=torch.bfloat16)
    keep("fused_output", y=y, S_final=sf)
    o = ex["o"].to(dev)
    keep("output", y=gdn2.output_fwd(o, g, wt, 1e-6), **gdn2.output_bwd(o, g, wt, 1e-6, dy))

    print("case decode step", flush=True)
    x = make_inputs(8, 1, 16, 128, 128, seed=9660, s0_std=0.1)
    d = {n: x[n][:, 0].contiguous().to(dev) for n in ("q", "k", "v", "log_alpha", "b", "w")}
    so, sn = gdn2.step(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], x["S0"].to(dev))
    keep("step", o=so, S=sn)
    torch.cuda.synchronize()
    torch.save(res, path)
    print("saved %d tensors" % len(res), flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
