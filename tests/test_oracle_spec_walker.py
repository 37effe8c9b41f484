"""Order fidelity of the oracle (CPU): a second evaluator of the row statistics, written
from the numerics' rules as a generic walker rather than per-layout loops, must give
the oracle's bits.

The walker takes the layout rule (W waves per row from H, P = 64W lanes, C chunks;
lane t owns the columns b*8P + 8t + v, visited b-major, v-minor), runs each lane's
ordered chain (RMS: s = RN(s + RN(x*x)); LN: Welford with the correctly rounded
reciprocal of the count), then one butterfly over all P lanes with distances 1, 2,
..., P/2, where at distance k lane t combines the partials of lanes t & ~k and t | k
in that order (the cross-wave pairs are the distances 64 and 128 of the same
butterfly), and finalizes with correctly rounded divide and square root.  All
arithmetic is numpy binary32 scalars, one rounding per operation.  Tiny H (8, 16, 64,
520) as the pin list asks, plus ragged two- and four-wave rows."""
import numpy as np
import pytest

from diffusion_dit_adaln_amd import synth
from oracle import oracle as O

F = np.float32
EPS32 = F(1e-6)


def layout(H):
    W = 1 if H < 2048 else 2 if H < 4096 else 4
    P = 64 * W
    return W, P, -(-H // (8 * P))


def lane_columns(H, t):
    _, P, C = layout(H)
    return [b * 8 * P + 8 * t + v for b in range(C) for v in range(8) if b * 8 * P + 8 * t + v < H]


def butterfly(parts, combine):
    P = len(parts)
    k = 1
    while k < P:
        parts = [combine(parts[t & ~k], parts[t | k]) for t in range(P)]
        k *= 2
    assert all(repr(p) == repr(parts[0]) for p in parts), "lanes disagree"
    return parts[0]


def rstd_of(stat, H):
    mean_sq = F(stat / F(H))
    v = F(mean_sq + EPS32)
    return F(F(1) / F(np.sqrt(v)))


def walk_rms(x):
    H = x.size
    _, P, _ = layout(H)
    parts = []
    for t in range(P):
        s = F(0)
        for c in lane_columns(H, t):
            s = F(s + F(x[c] * x[c]))
        parts.append(s)
    S = butterfly(parts, lambda a, b: F(a + b))
    return S, rstd_of(S, H)


def welford_combine(lo, hi):
    na, ma, qa = lo
    nb, mb, qb = hi
    if nb == 0:
        return lo
    if na == 0:
        return hi
    n = na + nb
    d = F(mb - ma)
    wb = F(F(nb) / F(n))
    m = F(ma + F(d * wb))
    q = F(F(qa + qb) + F(F(d * d) * F(F(na) * wb)))
    return (n, m, q)


def walk_ln(x):
    H = x.size
    _, P, _ = layout(H)
    parts = []
    for t in range(P):
        n, m, q = 0, F(0), F(0)
        for c in lane_columns(H, t):
            n += 1
            rho = F(F(1) / F(n))
            d = F(x[c] - m)
            m = F(m + F(d * rho))
            q = F(q + F(d * F(x[c] - m)))
        parts.append((n, m, q))
    n, m, q = butterfly(parts, welford_combine)
    assert n == H
    return m, q, rstd_of(q, H)


def rows_for(H, count, seed):
    rng = np.random.default_rng(seed)
    x = synth.normal_bf16(rng, (count, H))
    for i, sig in ((1, 1e-3), (2, 1e3)):
        x[i::3] = synth.normal_bf16(rng, x[i::3].shape, sig)
    x[0] = synth.f32_to_bf16_bits(np.zeros(H, np.float32))                 # zero row
    x[1] = synth.f32_to_bf16_bits(np.full(H, 3.0, np.float32))             # constant row
    onehot = np.zeros(H, np.float32)
    onehot[H // 2] = 1.0
    x[2] = synth.f32_to_bf16_bits(onehot)
    return x


@pytest.mark.parametrize("H,count", [(8, 60), (16, 60), (64, 40), (520, 20), (2056, 4),
                                     (4104, 3)])
def test_spec_walker_equals_oracle(H, count):
    x = rows_for(H, count, H)
    w = synth.normal_bf16(np.random.default_rng(7), (H,), 0.02, 1.0)
    z = np.zeros((1, H), np.uint16)
    _, yn_ln, st_ln = O.layernorm_modulate(x[None], z, z, 1e-6, want_norm=True, want_stats=True)
    _, yn_rms, st_rms = O.rmsnorm_scale_shift(x[None], w, z, z, 1e-6, want_norm=True,
                                              want_stats=True)
    wf = synth.bf16_bits_to_f32(w)
    for r in range(count):
        xf = synth.bf16_bits_to_f32(x[r])
        # RMS: statistic, rstd, and the norm output bf16(RN(RN(x*rstd)*RN(w+0)))
        S, rstd = walk_rms(xf)
        assert F(st_rms[r, 0]).tobytes() == S.tobytes(), (H, r, "S")
        assert F(st_rms[r, 4]).tobytes() == rstd.tobytes(), (H, r, "rms rstd")
        yn = np.array([F(F(xf[c] * rstd) * F(wf[c] + F(0))) for c in range(H)], np.float32)
        assert np.array_equal(synth.f32_to_bf16_bits(yn), yn_rms[0, r]), (H, r, "rms yn")
        # LN: mean, M2, rstd, and bf16(RN(RN(x-mean)*rstd))
        m, q, rstd = walk_ln(xf)
        assert F(st_ln[r, 0]).tobytes() == m.tobytes(), (H, r, "mean")
        assert F(st_ln[r, 1]).tobytes() == q.tobytes(), (H, r, "M2")
        assert F(st_ln[r, 5]).tobytes() == rstd.tobytes(), (H, r, "ln rstd")
        yn = np.array([F(F(xf[c] - m) * rstd) for c in range(H)], np.float32)
        assert np.array_equal(synth.f32_to_bf16_bits(yn), yn_ln[0, r]), (H, r, "ln yn")


def test_walker_catches_a_reversed_combine():
    # the walker is sensitive to the operand order it claims to follow: combining
    # (hi, lo) instead changes the bits of some of these rows
    _, P, _ = layout(64)
    differs = 0
    for xb in rows_for(64, 30, 3)[3:]:
        x = synth.bf16_bits_to_f32(xb)
        parts = []
        for t in range(P):
            n, m, q = 0, F(0), F(0)
            for c in lane_columns(64, t):
                n += 1
                d = F(x[c] - m)
                m = F(m + F(d * F(F(1) / F(n))))
                q = F(q + F(d * F(x[c] - m)))
            parts.append((n, m, q))
        fwd = butterfly(parts, welford_combine)
        k, rev = 1, parts
        while k < P:
            rev = [welford_combine(rev[t | k], rev[t & ~k]) for t in range(P)]
            k *= 2
        differs += (fwd[1].tobytes(), fwd[2].tobytes()) != (rev[0][1].tobytes(),
                                                             rev[0][2].tobytes())
    assert differs > 0
