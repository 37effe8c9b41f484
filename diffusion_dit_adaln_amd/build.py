"""Build libadaln.so in the package directory with hipcc for gfx950.

    python -m diffusion_dit_adaln_amd.build

Each source is compiled to an object on its own (in parallel), then linked.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, "adaln_kernels.hip"), os.path.join(CSRC, "adaln_qknorm.hip"),
           os.path.join(CSRC, "adaln_channel_first.hip"),
           os.path.join(CSRC, "adaln_stream.hip"), os.path.join(CSRC, "adaln_api.cpp")]
OUT = os.path.join(PKG, "libadaln.so")

# -ffp-contract=off: every fp32 add/mul rounds on its own (no FMA contraction).
# -packed-fp32-ops disabled: no v_pk_{add,mul,fma}_f32 are generated.
# Correctly rounded fp32 divide/sqrt are hipcc's default for '/' and sqrtf.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
               "-ffp-contract=off", "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "-Wall", "-Wno-unused-command-line-argument"]
_NOISE = "'-packed-fp32-ops' is not a recognized feature for this target"


def hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if _NOISE not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="adaln_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in SOURCES]
        jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            list(pool.map(lambda so: _run([hipcc(), *HIPCC_FLAGS, "-c", so[0], "-o", so[1]],
                                          verbose), zip(SOURCES, objs)))
        tmp = OUT + ".tmp"
        _run([hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", tmp], verbose)
        os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
