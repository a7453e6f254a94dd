"""The LDS poison-fill debug build (libgdn2_poison.so, compiled with -DGDN2_LDS_POISON): every
kernel first fills its whole LDS allocation with NaN words.  A kernel that reads a word of LDS
before writing it would then compute from NaN instead of whatever the CU's previous workgroup
left there, and its results would change.  Every kernel of the library runs on small seeded
cases (tests/lds_poison_cases.py: every launch path, gate format and pass) in a child process
with each build, and the two sets of results must be identical bit for bit.  The library is
chosen per process (GDN2_LIBRARY), hence the child processes.  The fused epilogue runs there on a
shape with one workgroup per head: the shapes with several take a cooperative launch, which the
runtime can refuse while another process on the GPU (this test's own) holds the device's
cooperative-launch resources."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
POISON = os.path.join(ROOT, "linear_attention_sequence_gdn2_amd", "libgdn2_poison.so")
NORMAL = os.path.join(ROOT, "linear_attention_sequence_gdn2_amd", "libgdn2.so")
CASES = os.path.join(ROOT, "tests", "lds_poison_cases.py")


def _run(lib, out):
    print("lds poison cases with %s" % os.path.basename(lib), flush=True)
    env = dict(os.environ, GDN2_LIBRARY=lib)
    p = subprocess.run([sys.executable, CASES, out], env=env, capture_output=True, text=True, timeout=110)
    print(p.stdout[-2000:], flush=True)
    assert p.returncode == 0, p.stderr[-3000:]
    return torch.load(out, weights_only=True)


@pytest.mark.gpu
def test_lds_poison_build_matches_normal_build(tmp_path):
    if not os.path.exists(POISON):
        pytest.skip("poison-fill library not built (python -m linear_attention_sequence_gdn2_amd.build --poison)")
    ref = _run(NORMAL, str(tmp_path / "normal.pt"))
    got = _run(POISON, str(tmp_path / "poison.pt"))
    assert set(ref) == set(got)
    assert len(ref) > 100
    diff = [n for n in ref if not torch.equal(ref[n], got[n])]
    assert not diff, diff
    nonfinite = [n for n in ref if ref[n].is_floating_point() and not bool(torch.isfinite(ref[n]).all())]
    assert not nonfinite, nonfinite
