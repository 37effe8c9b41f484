"""The entry points captured in a HIP graph: every replay recomputes the same bits
as the eager calls.  Outputs are cleared by eager work between the replays, so a
replay that skipped or reused a node would show."""
import numpy as np
import pytest
import torch

import diffusion_dit_adaln_amd as A
from diffusion_dit_adaln_amd import synth
from tests.helpers import dev, say

pytestmark = pytest.mark.gpu
EPS = 1e-6


def test_graph_replays_match_eager():
    say("[graph] capture all entry points, replay three times")
    rng = np.random.default_rng(21)
    B, T, H = 2, 300, 3072
    x = dev(synth.normal_bf16(rng, (B, T, H)))
    res = dev(synth.normal_bf16(rng, (B, T, H)))
    vec = [dev(synth.normal_bf16(rng, (B, H), 0.1)) for _ in range(3)]
    w = dev(synth.normal_bf16(rng, (H,), 0.02, 1.0))
    qs = torch.tensor([0.0125], dtype=torch.float32, device="cuda")
    qkv = dev(synth.normal_bf16(rng, (64, 3, 8, 128)))
    cs = torch.from_numpy(synth.rope_cache(64, 128)).cuda()
    Tc = 300                              # a ragged token count for the channel-first op
    res_cf = dev(synth.normal_bf16(rng, (B, H, Tc)))
    upd_cf = dev(synth.normal_bf16(rng, (B, Tc, H)))

    outs = {
        "ln": torch.empty_like(x), "rms": torch.empty_like(x), "rg_r": torch.empty_like(x),
        "rg_y": torch.empty_like(x), "rgln_r": torch.empty_like(x), "rgln_y": torch.empty_like(x),
        "q8": torch.empty(x.shape, dtype=torch.uint8, device="cuda"),
        "qo": torch.empty((64, 8, 128), dtype=torch.bfloat16, device="cuda"),
        "ko": torch.empty((64, 8, 128), dtype=torch.bfloat16, device="cuda"),
        "cf": torch.empty_like(res_cf),
    }

    def step(stream):
        A.adaln_layernorm_modulate(x, vec[0], vec[1], EPS, out=outs["ln"], stream=stream)
        A.adaln_rmsnorm_scale_shift(x, w, vec[0], vec[1], EPS, out=outs["rms"], stream=stream)
        A.adaln_residual_gate_rmsnorm_scale_shift(res, x, vec[2], w, vec[0], vec[1], EPS,
                                                  out=outs["rg_y"], r_out=outs["rg_r"],
                                                  stream=stream)
        A.adaln_residual_gate_layernorm_modulate(res, x, vec[2], vec[0], vec[1], EPS,
                                                 out=outs["rgln_y"], r_out=outs["rgln_r"],
                                                 stream=stream)
        A.adaln_layernorm_modulate_fp8_quant(x, vec[0], vec[1], qs, EPS, out=outs["q8"],
                                             stream=stream)
        A.adaln_qk_rmsnorm_rope(qkv[:, 0], qkv[:, 1], w[:128].contiguous(), None, cs, EPS,
                                q_out=outs["qo"], k_out=outs["ko"], stream=stream)
        A.adaln_residual_gate_channel_first(res_cf, upd_cf, vec[2], out=outs["cf"],
                                            stream=stream)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step(s)
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}

    for v in outs.values():
        v.zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for v in outs.values():
            v.fill_(7)                     # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v.view(torch.uint8), eager[k].view(torch.uint8)), (rep, k)
    del g
