"""Seeded random shapes for every op against the oracle, bit for bit (GPU).

Each case draws an op (LN, RMS with and without weight, residual-gate RMS with and
without weight, residual-gate LN, LN+FP8), a hidden size (any multiple of 8 up to
8192: one-, two- and four-wave rows, ragged last chunks), a batch split, a token
count (up to 12 M elements per tensor, and just past 2^25 for every op but LN+FP8,
so that every ring and row assignment of the launch plan and the one-shot grid come
up), the form of the per-batch vectors (one per
entry, one shared by the batch, or strided views of a wider embedding), eps and the
scale of the activations.  The case is printed before it runs."""
import numpy as np
import pytest
import torch

import diffusion_dit_adaln_amd as A
from diffusion_dit_adaln_amd import synth
from oracle import oracle as O
from tests.helpers import assert_bits_equal, dev, host, say

pytestmark = pytest.mark.gpu

OPS = ["ln", "rms", "rms_nw", "rg", "rg_nw", "rgln", "lnq"]
MAX_ELEMS = 3 << 20
N_CASES = 63


def draw(seed):
    """Three kinds of case, in turn over the ops: any hidden size up to 3 M elements;
    two- and four-wave rows up to 12 M elements; and, for every op but LN+FP8,
    launches just past 2^25 elements (the one-shot grid)."""
    rng = np.random.default_rng(seed)
    op = OPS[seed % len(OPS)]
    mode = (seed // len(OPS)) % 3
    B = int(rng.choice([1, 1, 2, 3, 5]))
    if mode == 0:
        H = max(8, min(8192, int(8 * round(2 ** rng.uniform(0, 10)))))
        T = int(rng.integers(1, max(2, MAX_ELEMS // (B * H))))
    elif mode == 1 or op == "lnq":
        H = 8 * int(rng.integers(256, 1025))
        T = int(rng.integers(1, max(2, 4 * MAX_ELEMS // (B * H))))
    else:
        H = 8 * int(rng.integers(128, 1025))
        B = int(rng.choice([1, 2, 3]))
        T = -(-((1 << 25) + int(rng.integers(0, 1 << 20))) // (B * H))
    vec = str(rng.choice(["per_entry", "shared", "strided"]))
    eps = float(rng.choice([1e-6, 1e-5, 0.0, 0.25]))
    sigma = float(rng.choice([1.0, 1e-3, 1e3]))
    return op, B, T, H, vec, eps, sigma, rng


def vectors(rng, B, H, kind, n):
    """n per-batch vectors as (host numpy, device tensor) pairs."""
    out = []
    if kind == "strided":
        emb = synth.normal_bf16(rng, (B, (n + 1) * H), 0.1)
        d = dev(emb)
        for i in range(n):
            out.append((emb[:, (i + 1) * H:(i + 2) * H], d[:, (i + 1) * H:(i + 2) * H]))
        return out
    rows = 1 if kind == "shared" else B
    for _ in range(n):
        v = synth.normal_bf16(rng, (rows, H), 0.1)
        out.append((v, dev(v)))
    return out


def oracle(op, x, res, g, w, sc, sh, eps, qscale):
    """The oracle's outputs (a tuple) of one op."""
    if op == "ln":
        return (O.layernorm_modulate(x, sc, sh, eps),)
    if op in ("rms", "rms_nw"):
        return (O.rmsnorm_scale_shift(x, w, sc, sh, eps),)
    if op in ("rg", "rg_nw"):
        return tuple(O.residual_gate_rmsnorm_scale_shift(res, x, g, w, sc, sh, eps))
    if op == "rgln":
        return tuple(O.residual_gate_layernorm_modulate(res, x, g, sc, sh, eps))
    return (O.layernorm_modulate_fp8(x, sc, sh, qscale, eps),)


def device(op, x, res, g, w, sc, sh, eps, qscale):
    """The device's outputs (a tuple of numpy arrays) of one op."""
    if op == "ln":
        return (host(A.adaln_layernorm_modulate(x, sc, sh, eps)),)
    if op in ("rms", "rms_nw"):
        return (host(A.adaln_rmsnorm_scale_shift(x, w, sc, sh, eps)),)
    if op in ("rg", "rg_nw"):
        return tuple(host(t) for t in A.adaln_residual_gate_rmsnorm_scale_shift(res, x, g, w, sc,
                                                                                  sh, eps))
    if op == "rgln":
        return tuple(host(t) for t in A.adaln_residual_gate_layernorm_modulate(res, x, g, sc, sh,
                                                                                 eps))
    qs = torch.tensor([qscale], dtype=torch.float32, device="cuda")
    return (A.adaln_layernorm_modulate_fp8_quant(x, sc, sh, qs, eps).cpu().numpy(),)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape(seed):
    op, B, T, H, vk, eps, sigma, rng = draw(seed)
    say(f"[random] seed={seed} op={op} B={B} T={T} H={H} vectors={vk} eps={eps} sigma={sigma}")
    x = synth.normal_bf16(rng, (B, T, H), sigma)
    res = synth.normal_bf16(rng, (B, T, H), sigma) if op in ("rg", "rg_nw", "rgln") else x
    (sc, scd), (sh, shd), (g, gd) = vectors(rng, B, H, vk, 3)
    w = synth.normal_bf16(rng, (H,), 0.02, 1.0) if op in ("rms", "rg") else None
    qscale = float(rng.choice([0.0125, 1.0, 3e-3, 40.0]))
    got = device(op, dev(x), dev(res), gd, None if w is None else dev(w), scd, shd, eps, qscale)
    if B * T * H <= 16 << 20:
        want = oracle(op, x, res, g, w, sc, sh, eps, qscale)
        for u, v in zip(got, want):
            assert_bits_equal(u, v, f"seed {seed}")
        return
    # large: 512 sampled rows, each with its own batch entry's vectors, as [n, 1, H]
    rows = np.sort(np.random.default_rng(seed).choice(B * T, size=512, replace=False))
    b = rows // T
    per_row = lambda v: np.ascontiguousarray(v[b if v.shape[0] == B else np.zeros_like(b)])
    xs = x.reshape(B * T, H)[rows][:, None]
    rs = res.reshape(B * T, H)[rows][:, None]
    want = oracle(op, xs, rs, per_row(g), w, per_row(sc), per_row(sh), eps, qscale)
    for u, v in zip(got, want):
        assert_bits_equal(u.reshape(B * T, H)[rows][:, None], v, f"seed {seed} (sampled)")


@pytest.mark.parametrize("seed", range(24))
def test_random_qk(seed):
    """QK-norm+RoPE: random token counts, Q and K head counts (either side may be
    absent), packed-QKV strided views or contiguous tensors, weights present or not,
    eps and scales."""
    rng = np.random.default_rng(5000 + seed)
    T = int(rng.integers(1, 9000))
    hq, hk = int(rng.integers(0, 49)), int(rng.integers(0, 49))
    if hq + hk == 0:
        hq = 1
    eps = float(rng.choice([1e-6, 1e-5, 0.25]))
    sigma = float(rng.choice([1.0, 1e-3, 1e3]))
    packed = bool(rng.integers(0, 2))
    say(f"[random] qk seed={seed} T={T} hq={hq} hk={hk} packed={packed} eps={eps} sigma={sigma}")
    if packed:
        hmax = max(hq, hk)
        qkv = synth.normal_bf16(rng, (T, 3, hmax, 128), sigma)
        d = dev(qkv)
        q, k = qkv[:, 0, :hq], qkv[:, 1, :hk]
        qd, kd = d[:, 0, :hq], d[:, 1, :hk]
    else:
        q, k = synth.normal_bf16(rng, (T, hq, 128), sigma), synth.normal_bf16(rng, (T, hk, 128), sigma)
        qd, kd = dev(q), dev(k)
    wq = synth.normal_bf16(rng, (128,), 0.02, 1.0) if rng.integers(0, 2) else None
    wk = synth.normal_bf16(rng, (128,), 0.02, 1.0) if rng.integers(0, 2) else None
    ang = rng.uniform(-np.pi, np.pi, (T, 64))
    cs = np.concatenate([np.cos(ang), np.sin(ang)], 1).astype(np.float32)
    qo, ko = A.adaln_qk_rmsnorm_rope(qd, kd, None if wq is None else dev(wq),
                                     None if wk is None else dev(wk), torch.from_numpy(cs).cuda(),
                                     eps)
    qo0, ko0 = O.qk_rmsnorm_rope(np.ascontiguousarray(q), np.ascontiguousarray(k), wq, wk, cs, eps)
    assert_bits_equal(host(qo), qo0, f"seed {seed} q")
    assert_bits_equal(host(ko), ko0, f"seed {seed} k")


@pytest.mark.parametrize("seed", range(24))
def test_random_channel_first(seed):
    """Channel-first residual gate: random batch, hidden (multiple of 8) and token
    counts (every residue mod 8 and mod 64), per-entry, shared or strided gates, out of
    place and in place."""
    rng = np.random.default_rng(7000 + seed)
    B = int(rng.choice([1, 2, 3]))
    H = 8 * int(rng.integers(1, 513))
    T = int(rng.integers(1, max(2, (4 << 20) // (B * H))))
    vk = str(rng.choice(["per_entry", "shared", "strided"]))
    in_place = bool(rng.integers(0, 2))
    say(f"[random] cf seed={seed} B={B} H={H} T={T} gate={vk} in_place={in_place}")
    res = synth.normal_bf16(rng, (B, H, T))
    upd = synth.normal_bf16(rng, (B, T, H))
    (g, gd), = vectors(rng, B, H, vk, 1)
    want = O.residual_gate_channel_first(res, upd, g)
    rd = dev(res)
    if in_place:
        A.adaln_residual_gate_channel_first(rd, dev(upd), gd, out=rd)
        got = rd
    else:
        got = A.adaln_residual_gate_channel_first(rd, dev(upd), gd)
    assert_bits_equal(host(got), want, f"seed {seed}")
