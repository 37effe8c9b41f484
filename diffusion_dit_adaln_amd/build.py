"""Build libadaln.so in the package directory with hipcc for gfx950.

    python -m diffusion_dit_adaln_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, "adaln_kernels.hip"), os.path.join(CSRC, "adaln_qknorm.hip"),
           os.path.join(CSRC, "adaln_channel_first.hip"), os.path.join(CSRC, "adaln_api.cpp")]
OUT = os.path.join(PKG, "libadaln.so")

# -ffp-contract=off: every fp32 add/mul rounds on its own (no FMA contraction).
# -packed-fp32-ops disabled: no v_pk_{add,mul,fma}_f32 are generated.
# Correctly rounded fp32 divide/sqrt are hipcc's default for '/' and sqrtf.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-ffp-contract=off", "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "-Wall", "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
