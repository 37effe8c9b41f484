"""The rings and row assignments the device plan chooses, checked against rows run
alone, against other plans of the same rows and against the oracle.

The plan of a launch comes from the device's own occupancy (adaln_diag_device_plan),
so each case first asserts which ring and assignment it exercises: the two-row ring
for four-wave RMS rows at the row counts where it spreads the groups more evenly, the
one-slot ring, the interleaved and contiguous assignments with one or many batch
entries, and the one-shot grid of large launches.  The same rows run as one [1, R, H] batch, as [R, 1, H] (B = R batch
entries of one row each), as two entries and one at a time must give the same bits:
batch invariance across plans as well as across launches (batch-invariance article,
section 3)."""
import numpy as np
import pytest
import torch

import diffusion_dit_adaln_amd as A
from diffusion_dit_adaln_amd import synth
from oracle import oracle as O
from tests.helpers import assert_bits_equal, dev, host, say

pytestmark = pytest.mark.gpu
EPS = 1e-6
QS = 0.0125


def mixed(rng, shape):
    """Rows of N(0,1), 1e-3 N(0,1) and 1e3 N(0,1) (the stress classes)."""
    x = synth.normal_bf16(rng, shape)
    R = int(np.prod(shape[:-1]))
    cls = rng.integers(0, 3, size=R)
    flat = x.reshape(R, -1)
    for c, sig in ((1, 1e-3), (2, 1e3)):
        idx = np.flatnonzero(cls == c)
        flat[idx] = synth.normal_bf16(rng, (idx.size, flat.shape[1]), sig)
    return x


def run(op, x, res, g, w, sc, sh, qs=None):
    """Outputs of one launch as a tuple of device tensors."""
    if op == "ln":
        return (A.adaln_layernorm_modulate(x, sc, sh, EPS),)
    if op == "rms":
        return (A.adaln_rmsnorm_scale_shift(x, w, sc, sh, EPS),)
    if op == "rg":
        return A.adaln_residual_gate_rmsnorm_scale_shift(res, x, g, w, sc, sh, EPS)
    if op == "rgln":
        return A.adaln_residual_gate_layernorm_modulate(res, x, g, sc, sh, EPS)
    return (A.adaln_layernorm_modulate_fp8_quant(x, sc, sh, qs, EPS),)


@pytest.mark.parametrize("op", ["ln", "rms", "rg", "rgln", "lnq"])
@pytest.mark.parametrize("H", [2048, 3072, 4096])
def test_plans_agree_on_the_same_rows(op, H):
    """[1, R, H], [R, 1, H], [2, R/2, H] and single rows give the same bits, although
    the launches differ: [R, 1, H] changes batch entry (and reloads its constants) at
    every row, [2, R/2, H] gives each entry its own share of the groups when the
    assignment is interleaved, a single row is a launch of one group."""
    R = 3000
    say(f"[paths] plans agree {op} H={H}")
    weight = op in ("rms", "rg")
    p1 = A.adaln_diag_device_plan(op, R, H, R, weight)
    p2 = A.adaln_diag_device_plan(op, R, H, R // 2, weight)
    if op in ("ln", "rgln", "lnq"):
        assert p2["gpb"] * 2 == p2["groups"] and p2["blk_rows"] == R // 2, (p1, p2)
    rng = np.random.default_rng(H + len(op))
    x = dev(mixed(rng, (R, H)))
    res = dev(mixed(rng, (R, H)))
    g = dev(synth.normal_bf16(rng, (1, H), 0.1))
    w = dev(synth.normal_bf16(rng, (H,), 0.02, 1.0)) if weight else None
    sc = dev(synth.normal_bf16(rng, (1, H), 0.1))
    sh = dev(synth.normal_bf16(rng, (1, H), 0.1))
    qs = torch.tensor([QS], dtype=torch.float32, device="cuda")
    a = run(op, x.view(1, R, H), res.view(1, R, H), g, w, sc, sh, qs)
    gR, scR, shR = (v.expand(R, H).contiguous() for v in (g, sc, sh))
    b = run(op, x.view(R, 1, H), res.view(R, 1, H), gR, w, scR, shR, qs)
    for u, v in zip(a, b):
        assert torch.equal(u.reshape(R, H).view(torch.uint8), v.reshape(R, H).view(torch.uint8))
    for r in (0, 1, 17, 1499, R - 1):
        c = run(op, x[r:r + 1].view(1, 1, H), res[r:r + 1].view(1, 1, H), g, w, sc, sh, qs)
        for u, v in zip(a, c):
            assert torch.equal(u[0, r].view(torch.uint8), v[0, 0].view(torch.uint8)), r
    d = run(op, x.view(2, R // 2, H), res.view(2, R // 2, H), g.expand(2, H).contiguous(), w,
            sc.expand(2, H).contiguous(), sh.expand(2, H).contiguous(), qs)
    for u, v in zip(a, d):
        assert torch.equal(u.reshape(R, H).view(torch.uint8), v.reshape(R, H).view(torch.uint8))
    # and the oracle on a sample of the rows
    rows = np.random.default_rng(2).choice(R, size=64, replace=False)
    idx = torch.from_numpy(rows).cuda()
    xs, rs = host(x[idx])[None], host(res[idx])[None]
    hv = [None if t is None else host(t) for t in (g, w, sc, sh)]
    if op == "ln":
        want = [O.layernorm_modulate(xs, hv[2], hv[3], EPS)]
    elif op == "rms":
        want = [O.rmsnorm_scale_shift(xs, hv[1], hv[2], hv[3], EPS)]
    elif op == "rg":
        want = list(O.residual_gate_rmsnorm_scale_shift(rs, xs, hv[0], hv[1], hv[2], hv[3], EPS))
    elif op == "rgln":
        want = list(O.residual_gate_layernorm_modulate(rs, xs, hv[0], hv[2], hv[3], EPS))
    else:
        want = [O.layernorm_modulate_fp8(xs, hv[2], hv[3], QS, EPS)]
    for u, wt in zip(a, want):
        picked = u[0][idx]
        got = picked.cpu().numpy() if op == "lnq" else host(picked)
        assert_bits_equal(got[None], wt, f"{op} H={H} sampled rows")


@pytest.mark.parametrize("H,weight", [(4096, True), (4096, False), (4104, True)])
def test_two_row_ring_rows_alone_and_in_batch(H, weight):
    """Four-wave RMS rows at a row count where the device plan picks the two-row ring
    (asserted first): every sampled row alone equals the row in the batch, and the
    batch equals the oracle."""
    T = None
    for rows in (8192, 5120, 10240, 4096, 3500, 6000, 7000, 9000):
        plan = A.adaln_diag_device_plan("rms", rows, H, rows, weight)
        if plan["ring"] == 2:
            T = rows
            break
    assert T is not None, "no row count takes the two-row ring on this device"
    assert plan["slots"] == 2 and not plan["shallow"]
    say(f"[paths] two-row ring rms T={T} H={H} weight={weight}")
    rng = np.random.default_rng(T + H)
    x = mixed(rng, (1, T, H))
    w = synth.normal_bf16(rng, (H,), 0.02, 1.0) if weight else None
    sc = synth.normal_bf16(rng, (1, H), 0.1)
    sh = synth.normal_bf16(rng, (1, H), 0.1)
    xd, scd, shd = dev(x), dev(sc), dev(sh)
    wd = None if w is None else dev(w)
    y = A.adaln_rmsnorm_scale_shift(xd, wd, scd, shd, EPS)
    assert_bits_equal(host(y), O.rmsnorm_scale_shift(x, w, sc, sh, EPS), f"rms {T}x{H}")
    for r in np.random.default_rng(1).choice(T, size=64, replace=False):
        y1 = A.adaln_rmsnorm_scale_shift(xd[:, r:r + 1].contiguous(), wd, scd, shd, EPS)
        assert torch.equal(y1[0, 0].view(torch.int16), y[0, r].view(torch.int16)), r


@pytest.mark.parametrize("op,rows,T,H,ring", [("rms", 2048, 2048, 4096, 1),
                                              ("ln", 9216, 4608, 3072, 1),
                                              ("ln", 4333, 4333, 3072, 0),
                                              ("rg", 2280, 1140, 4096, 0)])
def test_device_plan_rings(op, rows, T, H, ring):
    """The rings the configurations take on this device (the test above relies on the
    two-row ring; these pin the others): the one-slot ring for small four-wave RMS
    launches and for interleaved LayerNorm rows with three or more rows per group, the
    default depth otherwise."""
    plan = A.adaln_diag_device_plan(op, rows, H, T, op in ("rms", "rg"))
    assert plan["ring"] == ring, plan
    assert plan["resident"][0] >= 1 and plan["cus"] >= 1


def oracle_rows(op, xs, rs, g, w, sc, sh):
    """The oracle's outputs (a list) of one op on [1, n, H] rows with [1, H] vectors."""
    if op == "ln":
        return [O.layernorm_modulate(xs, sc, sh, EPS)]
    if op == "rms":
        return [O.rmsnorm_scale_shift(xs, w, sc, sh, EPS)]
    if op == "rg":
        return list(O.residual_gate_rmsnorm_scale_shift(rs, xs, g, w, sc, sh, EPS))
    return list(O.residual_gate_layernorm_modulate(rs, xs, g, sc, sh, EPS))


def assert_one_shot(plan, rows):
    S = plan["slots"]
    assert plan["ring"] == 0 and not plan["shallow"], plan
    assert (plan["span"], plan["group_stride"], plan["step"]) == (S, S, 1), plan
    assert plan["groups"] == -(-rows // S) > plan["resident"][0], plan


@pytest.mark.parametrize("op,B,T,H", [("rms", 1, 16384, 4096), ("rg", 2, 8191, 4096),
                                      ("rms", 1, 21846, 3072), ("rg", 1, 65536, 1024),
                                      ("rms", 1, 16353, 4104), ("rg", 1, 65028, 1032),
                                      ("ln", 1, 16384, 3072), ("rgln", 2, 8191, 3072),
                                      ("ln", 1, 32768, 1032), ("rgln", 1, 8192, 4104),
                                      ("ln", 3, 2731, 4096)])
def test_large_launches_take_the_one_shot_grid(op, B, T, H):
    """From 2^25 elements per launch every op but LN+FP8 takes the one-shot grid (one
    pass of the default ring per group, consecutive rows; asserted from the device
    plan first), with groups whose rows straddle two batch entries when T is not a
    multiple of the ring depth; sampled rows alone equal the rows in the batch, and
    both equal the oracle, the rows next to each entry boundary included."""
    rows = B * T
    weight = op in ("rms", "rg")
    plan = A.adaln_diag_device_plan(op, rows, H, T, weight)
    assert_one_shot(plan, rows)
    say(f"[paths] one-shot {op} B={B} T={T} H={H}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(rows + H)
    x = torch.randn((B, T, H), generator=gen, device="cuda").to(torch.bfloat16)
    res = torch.randn((B, T, H), generator=gen, device="cuda").to(torch.bfloat16)
    rng = np.random.default_rng(H)
    g = dev(synth.normal_bf16(rng, (B, H), 0.1))
    w = dev(synth.normal_bf16(rng, (H,), 0.02, 1.0)) if weight else None
    sc = dev(synth.normal_bf16(rng, (B, H), 0.1))
    sh = dev(synth.normal_bf16(rng, (B, H), 0.1))
    out = run(op, x, res, g, w, sc, sh)
    hv = [None if t is None else host(t) for t in (g, w, sc, sh)]
    for b in range(B):
        ts = np.unique(np.concatenate([[0, 1, 2, T - 3, T - 2, T - 1],
                                       np.random.default_rng(b).choice(T, size=32, replace=False)]))
        idx = torch.from_numpy(ts).cuda()
        vb = [None if t is None else t[b:b + 1] for t in (g, sc, sh)]
        for t in ts[:8]:  # alone
            alone = run(op, x[b:b + 1, t:t + 1].contiguous(), res[b:b + 1, t:t + 1].contiguous(),
                        vb[0], w, vb[1], vb[2])
            for u, v in zip(out, alone):
                assert torch.equal(u[b, t].view(torch.int16), v[0, 0].view(torch.int16)), (b, t)
        xs, rs = host(x[b][idx])[None], host(res[b][idx])[None]
        hb = [None if t is None else t[b:b + 1] for t in (hv[0], hv[2], hv[3])]
        want = oracle_rows(op, xs, rs, hb[0], hv[1], hb[1], hb[2])
        for u, wt in zip(out, want):
            assert_bits_equal(host(u[b][idx])[None], wt, f"{op} one-shot, entry {b}")


@pytest.mark.parametrize("op,H", [("rms", 1024), ("rg", 1024), ("rg", 4096), ("ln", 3072),
                                  ("rgln", 1024)])
def test_one_shot_every_row_its_own_entry(op, H):
    """The one-shot grid when every row is its own batch entry ([R, 1, H], per-row
    vectors, so a group reloads its constants at every row): sampled rows equal the
    oracle with their own vectors."""
    R = -(-(1 << 25) // H)
    weight = op in ("rms", "rg")
    plan = A.adaln_diag_device_plan(op, R, H, 1, weight)
    assert_one_shot(plan, R)
    say(f"[paths] one-shot [R,1,H] {op} R={R} H={H}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(R + H)
    x = torch.randn((R, 1, H), generator=gen, device="cuda").to(torch.bfloat16)
    res = torch.randn((R, 1, H), generator=gen, device="cuda").to(torch.bfloat16)
    vec = lambda: (0.1 * torch.randn((R, H), generator=gen, device="cuda")).to(torch.bfloat16)
    g, sc, sh = vec(), vec(), vec()
    w = dev(synth.normal_bf16(np.random.default_rng(H), (H,), 0.02, 1.0)) if weight else None
    out = run(op, x, res, g, w, sc, sh)
    wv = None if w is None else host(w)
    for r in np.random.default_rng(R).choice(R, size=48, replace=False):
        xs, rs = host(x[r:r + 1]), host(res[r:r + 1])
        gs, ss, hs = host(g[r:r + 1]), host(sc[r:r + 1]), host(sh[r:r + 1])
        want = oracle_rows(op, xs, rs, gs, wv, ss, hs)
        for u, wt in zip(out, want):
            assert_bits_equal(host(u[r:r + 1]), wt, f"{op} [R,1,{H}] row {r}")
