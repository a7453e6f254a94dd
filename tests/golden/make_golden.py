"""Write tests/golden/tiny_oracle_samples.json from the fp64 oracle.

The values are a regression fixture of the oracle itself (the pages print no
worked numerical example): any later change to the oracle's arithmetic must
reproduce them or explain, in its commit message, which reading of the pages
justifies the change.  Only the oracle and the seeded input generator are
called.  Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from linear_attention_sequence_gdn2_amd.inputs import WORKLOADS, make_workload  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle_samples.json")


def main():
    wl = WORKLOADS["tiny_f32_B1H2T128d32"]
    x = make_workload(wl, grads=True, s0_std=0.02)
    args = [x["q32"], x["k32"], x["v32"], x["log_alpha"], x["b"], x["w"], x["S0"]]
    o, sf = oracle.fwd(*args)
    g = oracle.bwd(*args, x["dO"], x["dS_final"])
    rng = np.random.default_rng(7)
    rec = {"workload": wl.name, "seed": wl.seed, "s0_std": 0.02, "grads": True,
           "source": "oracle/gdn2_oracle.c via tests/golden/make_golden.py", "samples": {}}
    for name, arr in [("o", o), ("S_final", sf)] + sorted(g.items()):
        idx = [tuple(int(i) for i in np.unravel_index(j, arr.shape))
               for j in rng.choice(arr.size, size=16, replace=False)]
        rec["samples"][name] = [[list(ix), float(arr[ix])] for ix in idx]
    with open(OUT, "w") as f:
        json.dump(rec, f, separators=(",", ":"))
        f.write("\n")
    print("wrote", OUT)


if __name__ == "__main__":
    main()
