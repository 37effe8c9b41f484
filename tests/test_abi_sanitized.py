"""The C-ABI's validation and launch planning under host sanitizers: the library's
sources are built with AddressSanitizer and UndefinedBehaviorSanitizer on their host
code (the device code is unchanged) and linked into tests/abi_fuzz_harness.cpp, which
calls every check predicate and the plan diagnostic some four million times with
random and boundary arguments.  Signed overflow, out-of-bounds access or any other
report fails the test.  Host only: nothing is launched."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "diffusion_dit_adaln_amd", "csrc")
SOURCES = ["adaln_api.cpp", "adaln_kernels.hip", "adaln_qknorm.hip", "adaln_channel_first.hip",
           "adaln_stream.hip"]
# sanitizers on the host side only, each right after -Xarch_host
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-ffp-contract=off", "-Xclang",
         "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    path = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return path if os.path.exists(path) else shutil.which("hipcc")


def test_validation_and_planning_under_host_sanitizers(tmp_path):
    cc = hipcc()
    if cc is None:
        pytest.skip("no hipcc")
    objs = []

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([cc, *FLAGS, *SAN, "-I", os.path.join(ROOT, "include"), "-c", src,
                            "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [os.path.join(HERE, "abi_fuzz_harness.cpp")]
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as pool:
        objs = list(pool.map(compile_one, srcs))
    exe = str(tmp_path / "abi_fuzz")
    r = subprocess.run([cc, "--offload-arch=gfx950", *SAN[:4], *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-4000:]
    assert "calls 2000000" in r.stdout
