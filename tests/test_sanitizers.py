"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU).

* The fp64 oracle (oracle/gdn2_oracle.c), built with gcc and the sanitizers, on small cases:
  ragged T across its 64-token checkpoints, several threads, optional arguments absent.
* The host side of the C ABI (csrc/gdn2_api.cpp, csrc/gdn2_noalloc.cpp), built with hipcc and
  the sanitizers on the host code only (-fno-gpu-sanitize), linked with the library's kernel
  objects, on every path that needs no GPU: buffer and workspace sizes, each argument check that
  refuses a call before any launch, the status strings.
Either run must exit 0 with no sanitizer report."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_sequence_gdn2_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")


def _run(exe):
    p = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    print(p.stdout[-3000:], p.stderr[-3000:])
    assert p.returncode == 0, p.stderr[-3000:]
    assert "Sanitizer" not in p.stderr and "runtime error" not in p.stderr


def test_oracle_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_asan")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c99", "-pthread"] + SAN +
                          ["-o", exe, os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                           os.path.join(ROOT, "oracle", "gdn2_oracle.c"), "-lm"])
    _run(exe)


def test_abi_host_checks_under_sanitizers():
    from linear_attention_sequence_gdn2_amd import build as hip_build
    kernels = [os.path.join(hip_build.BUILD_DIR, s + ".o") for s in hip_build.SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(k) for k in kernels):
        hip_build.build()
    os.makedirs(OUT, exist_ok=True)
    hipcc = hip_build.HIPCC
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", hip_build.INCLUDE, "-I", CSRC, "-fno-gpu-sanitize"] + SAN
    objs = []
    for src in (os.path.join(CSRC, "gdn2_api.cpp"), os.path.join(CSRC, "gdn2_noalloc.cpp"),
                os.path.join(ROOT, "tests", "sanitize", "api_driver.cpp")):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        subprocess.check_call([hipcc] + flags + ["-x", "hip", "-c", src, "-o", obj], stderr=subprocess.DEVNULL)
        objs.append(obj)
    exe = os.path.join(OUT, "api_asan")
    subprocess.check_call([hipcc, "-fno-gpu-sanitize", "--offload-arch=gfx950"] + SAN[:1] + objs + kernels +
                          ["-o", exe])
    _run(exe)
