"""The first call of a fresh process may come inside HIP graph capture.

A launcher's first call queries the device's occupancy for its kernels (cached
afterwards).  A caller that captures its denoise step before any eager call (FLUX
PR report, implementation item 2: the capture guard) makes those queries during
capture.  A child process therefore calls every entry point for the first time
inside a capture, replays the graph several times with eager work between the
replays, and compares every replay with the same calls made eagerly afterwards.
"""
import os
import subprocess
import sys

import pytest

from tests.helpers import say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, ROOT)
import numpy as np
import torch
import diffusion_dit_adaln_amd as A
from diffusion_dit_adaln_amd import synth

def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

rng = np.random.default_rng(8)
torch.cuda.init()
outs = {}
ins = {}
for H, T in ((3072, 300), (4096, 4216), (2048, 77)):
    B = 2
    ins[H] = dict(x=dev(synth.normal_bf16(rng, (B, T, H))), res=dev(synth.normal_bf16(rng, (B, T, H))),
                  v=[dev(synth.normal_bf16(rng, (B, H), 0.1)) for _ in range(3)],
                  w=dev(synth.normal_bf16(rng, (H,), 0.02, 1.0)))
    x = ins[H]["x"]
    for k in ("ln", "rms", "rg_r", "rg_y", "rgln_r", "rgln_y"):
        outs[(H, k)] = torch.empty_like(x)
    outs[(H, "q8")] = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
qs = torch.tensor([0.0125], dtype=torch.float32, device="cuda")
qkv = dev(synth.normal_bf16(rng, (64, 3, 8, 128)))
cs = torch.from_numpy(synth.rope_cache(64, 128)).cuda()
res_cf = dev(synth.normal_bf16(rng, (2, 3072, 4333)))
upd_cf = dev(synth.normal_bf16(rng, (2, 4333, 3072)))
g_cf = dev(synth.normal_bf16(rng, (2, 3072), 0.1))
outs["qo"] = torch.empty((64, 8, 128), dtype=torch.bfloat16, device="cuda")
outs["ko"] = torch.empty((64, 8, 128), dtype=torch.bfloat16, device="cuda")
outs["cf"] = torch.empty_like(res_cf)
torch.cuda.synchronize()

def step(s):
    for H, d in ins.items():
        x, res, (a, b, c), w = d["x"], d["res"], d["v"], d["w"]
        A.adaln_layernorm_modulate(x, a, b, 1e-6, out=outs[(H, "ln")], stream=s)
        A.adaln_rmsnorm_scale_shift(x, w, a, b, 1e-6, out=outs[(H, "rms")], stream=s)
        A.adaln_residual_gate_rmsnorm_scale_shift(res, x, c, w, a, b, 1e-6, out=outs[(H, "rg_y")],
                                                  r_out=outs[(H, "rg_r")], stream=s)
        A.adaln_residual_gate_layernorm_modulate(res, x, c, a, b, 1e-6, out=outs[(H, "rgln_y")],
                                                 r_out=outs[(H, "rgln_r")], stream=s)
        A.adaln_layernorm_modulate_fp8_quant(x, a, b, qs, 1e-6, out=outs[(H, "q8")], stream=s)
    A.adaln_qk_rmsnorm_rope(qkv[:, 0], qkv[:, 1], None, None, cs, 1e-6, q_out=outs["qo"],
                            k_out=outs["ko"], stream=s)
    A.adaln_residual_gate_channel_first(res_cf, upd_cf, g_cf, out=outs["cf"], stream=s)

s = torch.cuda.Stream()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g, stream=s):
    step(s)                      # the first library calls of this process
torch.cuda.synchronize()
replays = []
for rep in range(3):
    for v in outs.values():
        v.fill_(3)               # eager work between the replays
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    replays.append({k: v.clone() for k, v in outs.items()})
for v in outs.values():
    v.zero_()
torch.cuda.synchronize()
with torch.cuda.stream(s):
    step(s)
torch.cuda.synchronize()
for rep, got in enumerate(replays):
    for k, v in outs.items():
        assert torch.equal(got[k].view(torch.uint8), v.view(torch.uint8)), (rep, k)
del g
print("FIRST_CALL_IN_CAPTURE_OK", flush=True)
"""


def test_first_call_inside_graph_capture():
    say("[graph] child process: first library calls inside a capture")
    env = dict(os.environ)
    r = subprocess.run([sys.executable, "-c", f"ROOT = {ROOT!r}\n" + CHILD], env=env,
                       capture_output=True, text=True, timeout=300)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, f"child exited with {r.returncode}:\n{tail}"
    assert "FIRST_CALL_IN_CAPTURE_OK" in r.stdout, tail
