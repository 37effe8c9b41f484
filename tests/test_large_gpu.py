"""Maximum sizes: activations of more than 2^31 elements (over 4 GiB each), so that
every op of the fused kernel forms row addresses past 32 bits (the ERNIE-Image
RMSNorm+scale/shift report, implementation breakdown, widens its row index to 64
bits for the same reason).  Rows are independent and their arithmetic order depends
on H only, so the oracle run on sampled rows alone (the first, the last, the rows
on both sides of element 2^31, random ones) gives those rows' exact expected bits."""
import numpy as np
import pytest
import torch

import diffusion_dit_adaln_amd as A
from diffusion_dit_adaln_amd import synth
from oracle import oracle as O
from tests.helpers import assert_bits_equal, host, say

pytestmark = pytest.mark.gpu
EPS = 1e-6


def _draw(shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    t = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    flat = t.view(-1, shape[-1])
    for lo in range(0, flat.shape[0], 1 << 16):
        hi = min(flat.shape[0], lo + (1 << 16))
        flat[lo:hi] = torch.randn((hi - lo, shape[-1]), generator=g, device="cuda").to(
            torch.bfloat16)
    return t


@pytest.mark.parametrize("op,H", [("ln", 3072), ("rms", 4096), ("rg", 4096), ("rgln", 3072),
                                  ("lnq", 3072)])
def test_rows_past_two_to_the_31_elements(op, H):
    T = (1 << 31) // H + 20000          # > 2^31 elements, > 4 GiB per bf16 tensor
    say(f"[large] {op} [1,{T},{H}] ({T * H * 2 / 2**30:.1f} GiB per tensor)")
    x = _draw((1, T, H), 1)
    rng = np.random.default_rng(2)
    sc_h = synth.normal_bf16(rng, (1, H), 0.1)
    sh_h = synth.normal_bf16(rng, (1, H), 0.1)
    g_h = synth.normal_bf16(rng, (1, H), 0.1)
    w_h = synth.normal_bf16(rng, (H,), 0.02, 1.0)
    d = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    sc, sh, g, w = d(sc_h), d(sh_h), d(g_h), d(w_h)
    res = _draw((1, T, H), 3) if op in ("rg", "rgln") else None
    qs = torch.tensor([0.0125], dtype=torch.float32, device="cuda")
    if op == "ln":
        y = A.adaln_layernorm_modulate(x, sc, sh, EPS)
    elif op == "rms":
        y = A.adaln_rmsnorm_scale_shift(x, w, sc, sh, EPS)
    elif op == "rg":
        r, y = A.adaln_residual_gate_rmsnorm_scale_shift(res, x, g, w, sc, sh, EPS)
    elif op == "rgln":
        r, y = A.adaln_residual_gate_layernorm_modulate(res, x, g, sc, sh, EPS)
    else:
        y = A.adaln_layernorm_modulate_fp8_quant(x, sc, sh, qs, EPS)
    torch.cuda.synchronize()
    first_big = (1 << 31) // H + 1                                   # first row past 2^31
    rows = np.unique(np.concatenate([[0, 1, first_big - 1, first_big, T - 2, T - 1],
                                     rng.choice(T, 200, replace=False)]))
    idx = torch.from_numpy(rows).cuda()
    xs = host(x[0, idx])[None]
    if op == "ln":
        want = O.layernorm_modulate(xs, sc_h, sh_h, EPS)
    elif op == "rms":
        want = O.rmsnorm_scale_shift(xs, w_h, sc_h, sh_h, EPS)
    elif op == "rg":
        r0, want = O.residual_gate_rmsnorm_scale_shift(host(res[0, idx])[None], xs, g_h, w_h,
                                                       sc_h, sh_h, EPS)
        assert_bits_equal(host(r[0, idx])[None], r0, f"{op} r")
    elif op == "rgln":
        r0, want = O.residual_gate_layernorm_modulate(host(res[0, idx])[None], xs, g_h, sc_h,
                                                      sh_h, EPS)
        assert_bits_equal(host(r[0, idx])[None], r0, f"{op} r")
    else:
        want = O.layernorm_modulate_fp8(xs, sc_h, sh_h, 0.0125, EPS)
        got = y[0, idx].cpu().numpy()[None]
        assert np.array_equal(got, want), op
        return
    assert_bits_equal(host(y[0, idx])[None], want, op)
