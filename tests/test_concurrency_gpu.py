"""Concurrent use of the library (GPU): host threads launching different entry points on
streams of their own at the same time, and launches interleaved over two streams of
one thread, give the same bits as one-at-a-time launches.  The library keeps no state
between calls except its per-kernel occupancy cache (guarded by a mutex); the threads
make the test's first calls, so (run on its own) they race on filling it."""
import threading

import numpy as np
import pytest
import torch

import diffusion_dit_adaln_amd as A
from diffusion_dit_adaln_amd import synth
from tests.helpers import dev, host, say

pytestmark = pytest.mark.gpu
EPS = 1e-6


def make_cases():
    rng = np.random.default_rng(11)
    cases = []
    for op, (B, T, H) in (("ln", (2, 700, 3072)), ("rms", (1, 900, 4096)), ("rg", (2, 300, 4096)),
                          ("rgln", (1, 500, 2048)), ("lnq", (2, 400, 3072)),
                          ("rms", (1, 1 << 14, 4096)), ("ln", (1, 3000, 1024))):
        x, res = dev(synth.normal_bf16(rng, (B, T, H))), dev(synth.normal_bf16(rng, (B, T, H)))
        g, sc, sh = (dev(synth.normal_bf16(rng, (B, H), 0.1)) for _ in range(3))
        w = dev(synth.normal_bf16(rng, (H,), 0.02, 1.0))
        cases.append((op, x, res, g, w, sc, sh))
    cf = (dev(synth.normal_bf16(rng, (2, 3072, 777))), dev(synth.normal_bf16(rng, (2, 777, 3072))),
          dev(synth.normal_bf16(rng, (2, 3072), 0.1)))
    return cases, cf


def launch(case, stream):
    op, x, res, g, w, sc, sh = case
    if op == "ln":
        return (A.adaln_layernorm_modulate(x, sc, sh, EPS, stream=stream),)
    if op == "rms":
        return (A.adaln_rmsnorm_scale_shift(x, w, sc, sh, EPS, stream=stream),)
    if op == "rg":
        return A.adaln_residual_gate_rmsnorm_scale_shift(res, x, g, w, sc, sh, EPS, stream=stream)
    if op == "rgln":
        return A.adaln_residual_gate_layernorm_modulate(res, x, g, sc, sh, EPS, stream=stream)
    qs = torch.tensor([0.0125], dtype=torch.float32, device="cuda")
    return (A.adaln_layernorm_modulate_fp8_quant(x, sc, sh, qs, EPS, stream=stream),)


def bits(outs):
    return [o.cpu().numpy() if o.dtype == torch.uint8 else host(o) for o in outs]


def test_threads_on_their_own_streams():
    cases, cf = make_cases()
    torch.cuda.synchronize()
    say("[concurrency] 8 threads x 6 rounds")
    results, errors = {}, []

    def worker(t):
        try:
            s = torch.cuda.Stream()  # default priority
            outs = []
            for rnd in range(6):
                c = cases[(t + rnd) % len(cases)]
                with torch.cuda.stream(s):
                    o = launch(c, s)
                    ocf = A.adaln_residual_gate_channel_first(*cf, stream=s)
                outs.append(((t + rnd) % len(cases), o, ocf))
            s.synchronize()
            results[t] = [(i, bits(o), host(ocf)) for i, o, ocf in outs]
        except Exception as e:  # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not errors, errors
    assert len(results) == 8
    # the references only now, one launch at a time on the default stream, so that
    # the threads' first calls were the first of the test
    ref = [bits(launch(c, None)) for c in cases]
    ref_cf = host(A.adaln_residual_gate_channel_first(*cf))
    for t, outs in results.items():
        for i, got, got_cf in outs:
            for u, v in zip(got, ref[i]):
                assert np.array_equal(u, v), (t, i)
            assert np.array_equal(got_cf, ref_cf), t


def test_two_streams_interleaved():
    cases, _ = make_cases()
    torch.cuda.synchronize()
    ref = [bits(launch(c, None)) for c in cases]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for rnd in range(4):
        for i, c in enumerate(cases):
            s = s1 if (i + rnd) % 2 else s2
            with torch.cuda.stream(s):
                outs.append((i, launch(c, s)))
    torch.cuda.synchronize()
    for i, o in outs:
        for u, v in zip(bits(o), ref[i]):
            assert np.array_equal(u, v), i
