"""The instrumented build (libgdn2_stamps.so, compiled with -DGDN2_STAMPS): its clock stamps and its
GEMM-phase microkernels give the benchmark's per-phase figures.  The library is chosen per process
(GDN2_LIBRARY), so the measurement runs in a child process, as the benchmark runs it; these tests
check that every phase reports and that the figures are consistent with the kernels' structure."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "linear_attention_sequence_gdn2_amd", "libgdn2_stamps.so")

# B8 T2048 H16 dk = dv = 128: 4096 (batch, head, chunk) items; the sweep runs 256 workgroups of
# 64 value columns over 32 chunks each
ITEMS, SWEEP_WINDOWS = 8 * 16 * 32, 8 * 16 * 2 * 32
FORWARD_PHASES = {"a5 A,P": ITEMS, "a6 solve": ITEMS, "a7 X,QtS": SWEEP_WINDOWS, "a7 U=TX": SWEEP_WINDOWS,
                  "a7 O": SWEEP_WINDOWS, "a7 S'": SWEEP_WINDOWS}
CHUNK_PHASES = ("record into LDS", "value tile 0", "value tile 1", "value tiles 2-3", "epilogue inputs",
                "dP/dA products and chain", "dlog_alpha scans and stores")


@pytest.fixture(scope="module")
def phases():
    if not os.path.exists(LIB):
        pytest.skip("instrumented library not built (python -m linear_attention_sequence_gdn2_amd.build --stamps)")
    print("instrumented build: bench.py --phase-stamps in a child process", flush=True)
    env = dict(os.environ, GDN2_LIBRARY=LIB)
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--phase-stamps"], env=env,
                       capture_output=True, text=True, timeout=110)
    assert p.returncode == 0, p.stderr[-3000:]
    return json.loads(p.stdout.strip().splitlines()[-1])


def _frac_ok(ph):
    # executed MFMA use is a fraction of the per-CU peak; useful (one MFMA per split product)
    # is at most the executed figure
    assert 0.0 < ph["executed_frac"] <= 1.0, ph
    assert 0.0 < ph["useful_frac"] <= ph["executed_frac"], ph
    assert ph["window_cycles_mean"] > 0, ph


@pytest.mark.gpu
def test_forward_phase_stamps(phases):
    assert set(phases["phases"]) == set(FORWARD_PHASES)
    for name, windows in FORWARD_PHASES.items():
        ph = phases["phases"][name]
        assert ph["windows"] == windows, (name, ph)
        _frac_ok(ph)
        assert 0.0 < ph["share_of_launch_cycles"] < 1.0, (name, ph)
    # a window runs from the first wave entering to the last leaving, so consecutive windows of one
    # kernel overlap a little and their shares may add up to somewhat more than the launch
    for kern in ("bwd_factors_kernel (forward-only records)", "fwd_sweep64_kernel"):
        share = sum(p["share_of_launch_cycles"] for p in phases["phases"].values() if p["kernel"] == kern)
        assert 0.3 < share <= 1.3, (kern, share)
    g = phases["gemm_phases"]
    assert 0.0 < g["useful_frac"] <= g["executed_frac"] <= 1.0
    assert g["gap_to_target_executed"] == pytest.approx(0.40 - g["executed_frac"], abs=1e-3)


@pytest.mark.gpu
def test_chunk_gradient_phase_stamps(phases):
    c = phases["chunk_gradient_phases"]
    assert c["items"] == ITEMS and c["item_cycles_mean"] > 0
    assert set(c["phases"]) == set(CHUNK_PHASES)
    for name in CHUNK_PHASES:
        assert 0.0 < c["phases"][name]["share"] < 1.0, (name, c["phases"][name])
    # the phases follow one another inside an item: their windows (overlapping a little, as above)
    # add up to about the item
    total = sum(p["share"] for p in c["phases"].values())
    assert 0.9 <= total <= 1.2, total


@pytest.mark.gpu
def test_resident_microkernels(phases):
    r = phases["resident_microkernel"]
    assert set(r["phases"]) == set(FORWARD_PHASES)
    for name, ph in r["phases"].items():
        _frac_ok(ph)
    # with no memory traffic in the window, each phase runs at least as fast as inside the
    # memory-bound kernels
    for name in FORWARD_PHASES:
        assert r["phases"][name]["window_cycles_mean"] < phases["phases"][name]["window_cycles_mean"] * 1.05, name
