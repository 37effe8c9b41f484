"""GPU parity: the HIP path through the C ABI equals the CPU oracle bit for bit.

Sizes: the five workloads at their full sizes (the oracle finishes each in
seconds), the FLUX.1 site signatures with strided `emb.chunk` modulation views
(FLUX PR report, test snippet), ragged and extreme hidden sizes, empty and
single-row inputs, non-finite inputs, and exhaustive sweeps of the device's
bf16 rounding and finalize steps.
"""
import numpy as np
import pytest
import torch

import diffusion_dit_adaln_amd as A
from diffusion_dit_adaln_amd import synth
from oracle import oracle as O
from tests.helpers import assert_bits_equal, dev, host, say

pytestmark = pytest.mark.gpu
EPS = 1e-6


def run_ln(x, sc, sh, eps=EPS):
    return host(A.adaln_layernorm_modulate(dev(x), dev(sc), dev(sh), eps))


def run_rms(x, w, sc, sh, eps=EPS):
    return host(A.adaln_rmsnorm_scale_shift(dev(x), None if w is None else dev(w), dev(sc), dev(sh),
                                            eps))


def run_rg(res, x, g, w, sc, sh, eps=EPS):
    r, y = A.adaln_residual_gate_rmsnorm_scale_shift(dev(res), dev(x), dev(g),
                                                     None if w is None else dev(w), dev(sc),
                                                     dev(sh), eps)
    return host(r), host(y)


def run_rgln(res, x, g, sc, sh, eps=EPS):
    r, y = A.adaln_residual_gate_layernorm_modulate(dev(res), dev(x), dev(g), dev(sc), dev(sh), eps)
    return host(r), host(y)


def check_rgln(res, x, g, sc, sh, what, eps=EPS):
    r, y = run_rgln(res, x, g, sc, sh, eps)
    r0, y0 = O.residual_gate_layernorm_modulate(res, x, g, sc, sh, eps)
    assert_bits_equal(r, r0, what + " r")
    assert_bits_equal(y, y0, what + " y")


def run_lnq(x, sc, sh, qscale, eps=EPS):
    qs = torch.tensor([qscale], dtype=torch.float32, device="cuda")
    return A.adaln_layernorm_modulate_fp8_quant(dev(x), dev(sc), dev(sh), qs, eps).cpu().numpy()


def assert_fp8_equal(got, want, what):
    """E4M3 codes equal bit for bit, NaN codes (0xFF) included."""
    gn = (got & 0x7F) == 0x7F
    wn = (want & 0x7F) == 0x7F
    assert np.array_equal(gn, wn), what + ": NaN positions differ"
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{what}: {bad.size} codes differ, first at {bad[:5]}"


def assert_same_nans(got, want, what):
    """bf16 outputs equal bit for bit where finite; NaN in the same places, every NaN
    quiet on both sides.  The sign of a NaN is not part of the numerics (IEEE 754 does
    not interpret it): inf * 0 gives 0xFFC00000 on the host's SSE arithmetic and
    0x7FC00000 from gfx950's v_mul_f32."""
    gn = np.isnan(synth.bf16_bits_to_f32(got))
    wn = np.isnan(synth.bf16_bits_to_f32(want))
    assert np.array_equal(gn, wn), what + ": NaN positions differ"
    assert_bits_equal(got[~gn], want[~wn], what + " (finite outputs)")
    for a, who in ((got[gn], "device"), (want[wn], "oracle")):
        assert np.all((a & 0x7FC0) == 0x7FC0), f"{what}: a {who} NaN is not quiet"


def check_lnq(x, sc, sh, qscale, what, eps=EPS):
    assert_fp8_equal(run_lnq(x, sc, sh, qscale, eps),
                     O.layernorm_modulate_fp8(x, sc, sh, qscale, eps), what)


def check_workload(wl, what):
    say(f"[parity] {what} {wl.op} shape={wl.x.shape}")
    if wl.op == "ln":
        assert_bits_equal(run_ln(wl.x, wl.scale, wl.shift), O.layernorm_modulate(
            wl.x, wl.scale, wl.shift, wl.eps), what)
    elif wl.op == "rms":
        assert_bits_equal(run_rms(wl.x, wl.weight, wl.scale, wl.shift), O.rmsnorm_scale_shift(
            wl.x, wl.weight, wl.scale, wl.shift, wl.eps), what)
    elif wl.op == "lnq":
        check_lnq(wl.x, wl.scale, wl.shift, wl.qscale, what, wl.eps)
    elif wl.op == "rgln":
        check_rgln(wl.res, wl.x, wl.gate, wl.scale, wl.shift, what, wl.eps)
    else:
        r, y = run_rg(wl.res, wl.x, wl.gate, wl.weight, wl.scale, wl.shift)
        r0, y0 = O.residual_gate_rmsnorm_scale_shift(wl.res, wl.x, wl.gate, wl.weight, wl.scale,
                                                     wl.shift, wl.eps)
        assert_bits_equal(r, r0, what + " r")
        assert_bits_equal(y, y0, what + " y")


# --------------------------------------------------------------------------
# the workloads at full size
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["ln_1x128x2048", "rms_1x4216x4096", "rg_rms_2x1140x4096",
                                  "ln_2x4608x3072", "ln_1x4333x3072", "rg_ln_2x4096x3072",
                                  "ln_fp8_2x4608x3072"])
def test_workload_full_size(name):
    check_workload(synth.WORKLOADS[name](), name)


def test_rg_with_weight():
    wl = synth.rg_rms_2x1140x4096()
    wl.weight = synth.normal_bf16(np.random.default_rng(5), (4096,), 0.02, 1.0)
    check_workload(wl, "rg_rms_2x1140x4096 with weight")


# --------------------------------------------------------------------------
# FLUX.1 site signatures with strided modulation views
# --------------------------------------------------------------------------
@pytest.mark.parametrize("shape,chunks", [((1, 4096, 3072), 6), ((1, 512, 3072), 6),
                                          ((1, 4608, 3072), 3), ((2, 300, 3072), 6)])
def test_flux_sites_chunk_views(shape, chunks):
    B, T, H = shape
    say(f"[parity] flux site {shape} chunk({chunks})")
    rng = np.random.default_rng(0)
    x = synth.normal_bf16(rng, shape, 8.0)          # randn * 8, as in the test snippet
    emb, shift, scale = synth.flux_chunk_views(0, B, H, chunks)
    emb_d = dev(emb)
    shift_d = emb_d[:, 0:H]
    scale_d = emb_d[:, H:2 * H]
    assert scale_d.stride(0) == chunks * H
    y = host(A.adaln_layernorm_modulate(dev(x), scale_d, shift_d, EPS))
    assert_bits_equal(y, O.layernorm_modulate(x, scale, shift, EPS), f"flux {shape}")
    # the RMS variant through the same strided views
    y = host(A.adaln_rmsnorm_scale_shift(dev(x), None, scale_d, shift_d, EPS))
    assert_bits_equal(y, O.rmsnorm_scale_shift(x, None, scale, shift, EPS), f"flux rms {shape}")
    # the residual-gate LayerNorm with its gate a third slice of the same embedding
    res = synth.normal_bf16(rng, shape, 8.0)
    gate = emb[:, 2 * H:3 * H]
    r, y = A.adaln_residual_gate_layernorm_modulate(dev(res), dev(x), emb_d[:, 2 * H:3 * H],
                                                    scale_d, shift_d, EPS)
    r0, y0 = O.residual_gate_layernorm_modulate(res, x, gate, scale, shift, EPS)
    assert_bits_equal(host(r), r0, f"flux rgln r {shape}")
    assert_bits_equal(host(y), y0, f"flux rgln y {shape}")
    # the FP8 variant through the same strided views
    qs = torch.tensor([0.0125], dtype=torch.float32, device="cuda")
    q = A.adaln_layernorm_modulate_fp8_quant(dev(x), scale_d, shift_d, qs, EPS).cpu().numpy()
    assert_fp8_equal(q, O.layernorm_modulate_fp8(x, scale, shift, 0.0125, EPS), f"flux lnq {shape}")


# --------------------------------------------------------------------------
# hidden sizes: ragged tails, both layouts, the extremes
# --------------------------------------------------------------------------
EDGE_H = [8, 16, 24, 64, 504, 512, 520, 1000, 1536, 2040, 2048, 2056, 3064, 3072, 3080, 4088,
          4096, 4104, 5000, 6144, 8184, 8192]


def mixed_rows(rng, B, T, H):
    cls = rng.integers(0, 4, size=(B, T, 1))
    sig = np.array([1.0, 1e-3, 1e3, 8.0])[cls]
    mu = np.where(cls == 3, 100.0, 0.0)
    v = rng.standard_normal((B, T, H)) * sig + mu
    return synth.f32_to_bf16_bits(v.astype(np.float32)).reshape(B, T, H)


@pytest.mark.parametrize("H", EDGE_H)
def test_edge_hidden_sizes(H):
    say(f"[parity] edge H={H}")
    rng = np.random.default_rng(H)
    B, T = 2, 7
    x = mixed_rows(rng, B, T, H)
    res = mixed_rows(rng, B, T, H)
    w = synth.normal_bf16(rng, (H,), 0.02, 1.0)
    g = synth.normal_bf16(rng, (B, H), 0.1)
    sc = synth.normal_bf16(rng, (B, H), 0.1)
    sh = synth.normal_bf16(rng, (B, H), 0.1)
    assert_bits_equal(run_ln(x, sc, sh), O.layernorm_modulate(x, sc, sh, EPS), f"ln H={H}")
    for ww in (w, None):
        tag = f"H={H} weight={ww is not None}"
        assert_bits_equal(run_rms(x, ww, sc, sh), O.rmsnorm_scale_shift(x, ww, sc, sh, EPS),
                          "rms " + tag)
        r, y = run_rg(res, x, g, ww, sc, sh)
        r0, y0 = O.residual_gate_rmsnorm_scale_shift(res, x, g, ww, sc, sh, EPS)
        assert_bits_equal(r, r0, "rg r " + tag)
        assert_bits_equal(y, y0, "rg y " + tag)
    check_rgln(res, x, g, sc, sh, f"rgln H={H}")
    for qs in (0.0125, 1.0):
        check_lnq(x, sc, sh, qs, f"lnq H={H} qscale={qs}")


def _all_rows(alphabet, H, stride=1):
    a = synth.f32_to_bf16_bits(np.array(alphabet, np.float32))
    idx = np.indices((len(a),) * H).reshape(H, -1).T[::stride]
    return np.ascontiguousarray(a[idx])


# Brute force over small alphabets: every row of 8 values from six letters
# (1.68 M rows, the oracle's own brute-force pin), and every 27th row of 16 values
# from {-1, 0, 1} (1.59 M rows: ties, cancellations, zero rows, one-hot rows).
@pytest.mark.parametrize("H,alphabet,stride", [(8, [0.0, 0.5, -1.0, 2.0, -3.0, 0.0625], 1),
                                               (16, [-1.0, 0.0, 1.0], 27)])
def test_brute_force_rows(H, alphabet, stride):
    x = _all_rows(alphabet, H, stride)[None]
    say(f"[parity] brute force H={H} rows={x.shape[1]}")
    rng = np.random.default_rng(H)
    sc = synth.normal_bf16(rng, (1, H), 0.1)
    sh = synth.normal_bf16(rng, (1, H), 0.1)
    w = synth.normal_bf16(rng, (H,), 0.02, 1.0)
    assert_bits_equal(run_ln(x, sc, sh), O.layernorm_modulate(x, sc, sh, EPS), f"ln H={H}")
    assert_bits_equal(run_rms(x, w, sc, sh), O.rmsnorm_scale_shift(x, w, sc, sh, EPS),
                      f"rms H={H}")


@pytest.mark.parametrize("op", ["ln", "rms"])
def test_norm_outputs_near_torch_eager(op):
    """A loose cross-check against an implementation of another order (never a gate of
    the numerics): with zero modulation the outputs are the norm outputs, and they lie
    within 2 bf16 ulp of torch's own eager layer_norm / rms_norm computed in binary32 on
    the device and rounded to bf16 (for LayerNorm plus the floor of the mean's own
    error, as in the oracle's float64 pins)."""
    import torch.nn.functional as Fn

    from tests.test_oracle_pins import KAPPA, U32, ulp_bf16

    wl = synth.WORKLOADS["ln_2x4608x3072" if op == "ln" else "rms_1x4216x4096"]()
    B, T, H = wl.x.shape
    say(f"[parity] {op} against torch eager {wl.x.shape}")
    x = dev(wl.x)
    z = torch.zeros((B, H), dtype=torch.bfloat16, device="cuda")
    xf = x.float()
    if op == "ln":
        ours = A.adaln_layernorm_modulate(x, z, z, EPS)
        ref = Fn.layer_norm(xf, (H,), eps=EPS).to(torch.bfloat16)
        mu = xf.mean(dim=-1, keepdim=True)
        sd = (xf - mu).pow(2).mean(dim=-1, keepdim=True).sqrt()
        floor = (KAPPA * U32 * (mu.abs() + sd) / (sd + 1e-30)).double().cpu().numpy()
    else:
        w = dev(wl.weight)
        ours = A.adaln_rmsnorm_scale_shift(x, w, z, z, EPS)
        ref = Fn.rms_norm(xf, (H,), weight=w.float(), eps=EPS).to(torch.bfloat16)
        floor = 0.0
    a = synth.bf16_bits_to_f32(host(ours)).astype(np.float64)
    b = synth.bf16_bits_to_f32(host(ref)).astype(np.float64)
    tol = 2.0 * ulp_bf16(b) + floor
    bad = np.abs(a - b) > tol
    assert not bad.any(), (int(bad.sum()), float((np.abs(a - b) / tol).max()))
    say(f"[parity] {op}: {float((a == b).mean()):.4f} of the outputs equal torch's bit for bit")


@pytest.mark.parametrize("name", ["h8", "h16"])
def test_brute_force_full_domains(name):
    """Every row of 8 values over {0, +-0.5, +-1, +-2, 3} (16.8 M rows) and of 16
    values over {-1, 0, 1} (43 M rows): the device's LayerNorm+modulate and
    RMSNorm+scale/shift outputs, in row order, hash to the oracle's digests stored in
    tests/golden (written by a script that calls only the oracle; the CPU suite
    recomputes them from the oracle and checks them against the float64 definition)."""
    import hashlib

    from tests import brute_domains as D

    g = D.golden_digests()
    H, _ = D.DOMAINS[name]
    say(f"[parity] brute force {name}: {D.size(name)} rows of H={H}")
    sc, sh, w = (dev(v) for v in D.vectors(H))
    h_ln, h_rms = hashlib.sha256(), hashlib.sha256()
    for lo, hi in D.chunks(name):
        x = dev(D.rows(name, lo, hi)[None])
        h_ln.update(host(A.adaln_layernorm_modulate(x, sc, sh, EPS)).tobytes())
        h_rms.update(host(A.adaln_rmsnorm_scale_shift(x, w, sc, sh, EPS)).tobytes())
    assert h_ln.hexdigest() == g[(name, "ln")], "LayerNorm+modulate differs from the oracle"
    assert h_rms.hexdigest() == g[(name, "rms")], "RMSNorm+scale/shift differs from the oracle"


# Row counts large enough that the interleaved ops take their one-slot ring (at
# least three rows per resident row group), for one-, two- and four-wave rows with
# and without a ragged last chunk.
@pytest.mark.parametrize("op,T,H", [("ln", 30000, 520), ("ln", 30000, 1024),
                                    ("ln", 7000, 3080), ("ln", 3600, 4104),
                                    ("rgln", 30000, 1536), ("rgln", 6400, 2048),
                                    ("lnq", 4000, 4096), ("lnq", 30000, 776)])
def test_many_rows_per_group(op, T, H):
    say(f"[parity] many rows {op} T={T} H={H}")
    rng = np.random.default_rng(T + H)
    x = synth.normal_bf16(rng, (1, T, H))
    sc = synth.normal_bf16(rng, (1, H), 0.1)
    sh = synth.normal_bf16(rng, (1, H), 0.1)
    if op == "ln":
        assert_bits_equal(run_ln(x, sc, sh), O.layernorm_modulate(x, sc, sh, EPS), f"ln {T}x{H}")
    elif op == "rgln":
        res = synth.normal_bf16(rng, (1, T, H))
        g = synth.normal_bf16(rng, (1, H), 0.1)
        check_rgln(res, x, g, sc, sh, f"rgln {T}x{H}")
    else:
        check_lnq(x, sc, sh, 0.0125, f"lnq {T}x{H}")


# Several batch entries with enough rows for the one-slot ring: the interleaved ops
# then give each entry its own share of the row groups (rows per group uneven, e.g.
# 1500 rows over 365 groups), up to the split that leaves exactly 1/16 of the groups
# idle (300 entries of 40 rows), and past it one interleave over all rows whose groups
# change entry (1000 entries of 12 rows).  Each entry has its own vectors.
@pytest.mark.parametrize("op,B,T,H", [("ln", 7, 1500, 3072), ("lnq", 3, 3001, 2056),
                                      ("rgln", 2, 5000, 1024), ("ln", 40, 300, 3072),
                                      ("ln", 300, 40, 3072), ("ln", 1000, 12, 3072),
                                      ("rgln", 5, 2000, 4096)])
def test_batch_entries_split_over_groups(op, B, T, H):
    say(f"[parity] batch split {op} B={B} T={T} H={H}")
    rng = np.random.default_rng(B * 7919 + T + H)
    x = synth.normal_bf16(rng, (B, T, H))
    sc = synth.normal_bf16(rng, (B, H), 0.1)
    sh = synth.normal_bf16(rng, (B, H), 0.1)
    if op == "ln":
        assert_bits_equal(run_ln(x, sc, sh), O.layernorm_modulate(x, sc, sh, EPS),
                          f"ln {B}x{T}x{H}")
    elif op == "rgln":
        res = synth.normal_bf16(rng, (B, T, H))
        g = synth.normal_bf16(rng, (B, H), 0.1)
        check_rgln(res, x, g, sc, sh, f"rgln {B}x{T}x{H}")
    else:
        check_lnq(x, sc, sh, 0.0125, f"lnq {B}x{T}x{H}")


# RMS row counts where the four-wave rows take the two-row ring (the groups then
# spread more evenly over the CUs than with the three-row ring), with and without a
# ragged last chunk and the weight.
@pytest.mark.parametrize("T,H,weight", [(8192, 4096, True), (5120, 4096, False),
                                        (4096, 4104, True), (10240, 4096, True)])
def test_rms_two_row_ring_sizes(T, H, weight):
    say(f"[parity] rms two-row ring T={T} H={H} weight={weight}")
    rng = np.random.default_rng(T * 3 + H)
    x = synth.normal_bf16(rng, (1, T, H))
    w = synth.normal_bf16(rng, (H,), 0.02, 1.0) if weight else None
    sc = synth.normal_bf16(rng, (1, H), 0.1)
    sh = synth.normal_bf16(rng, (1, H), 0.1)
    assert_bits_equal(run_rms(x, w, sc, sh), O.rmsnorm_scale_shift(x, w, sc, sh, EPS),
                      f"rms {T}x{H}")


@pytest.mark.parametrize("eps", [0.0, 1e-5, 1e-6, 0.25])
def test_eps_values(eps):
    say(f"[parity] eps={eps}")
    rng = np.random.default_rng(17)
    for H in (3072, 4096):
        x = mixed_rows(rng, 1, 9, H)
        sc = synth.normal_bf16(rng, (1, H), 0.1)
        sh = synth.normal_bf16(rng, (1, H), 0.1)
        assert_bits_equal(run_ln(x, sc, sh, eps), O.layernorm_modulate(x, sc, sh, eps), "ln")
        assert_bits_equal(run_rms(x, None, sc, sh, eps), O.rmsnorm_scale_shift(x, None, sc, sh, eps),
                          "rms")
        res = mixed_rows(rng, 1, 9, H)
        g = synth.normal_bf16(rng, (1, H), 0.1)
        check_rgln(res, x, g, sc, sh, f"rgln eps={eps}", eps)
        check_lnq(x, sc, sh, 0.02, f"lnq eps={eps}", eps)


def test_constant_and_zero_rows():
    say("[parity] constant / zero / denormal rows")
    H = 4096
    consts = np.array([0.0, -0.0, 1.0, -3.5, 1e3, 2.0 ** -130, -(2.0 ** -133), 65504.0],
                      np.float32)
    x = np.repeat(synth.f32_to_bf16_bits(consts)[:, None], H, axis=1)[None]
    rng = np.random.default_rng(2)
    sc = synth.normal_bf16(rng, (1, H), 0.1)
    sh = synth.normal_bf16(rng, (1, H), 0.1)
    assert_bits_equal(run_ln(x, sc, sh), O.layernorm_modulate(x, sc, sh, EPS), "ln")
    assert_bits_equal(run_rms(x, None, sc, sh), O.rmsnorm_scale_shift(x, None, sc, sh, EPS), "rms")
    # residual gate with a zero gate: r is the constant residual row, y the shift
    upd = synth.normal_bf16(rng, x.shape)
    zero = np.zeros((1, H), np.uint16)
    check_rgln(x, upd, zero, sc, sh, "rgln zero gate")
    for qs in (0.0125, 1e-3, 2.0 ** -12):   # the last saturates most outputs at +-448
        check_lnq(x, sc, sh, qs, f"lnq constant rows qscale={qs}")


def test_nonfinite_inputs_give_nan_in_the_same_places():
    say("[parity] inf / nan inputs")
    H = 3072
    rng = np.random.default_rng(4)
    x = synth.normal_bf16(rng, (1, 6, H))
    x[0, 1, 7] = 0x7F80     # +inf
    x[0, 2, 100] = 0xFF80   # -inf
    x[0, 3, 2000] = 0x7FC0  # nan
    sc = synth.normal_bf16(rng, (1, H), 0.1)
    sh = synth.normal_bf16(rng, (1, H), 0.1)
    res = synth.normal_bf16(rng, (1, 6, H))
    res[0, 4, 9] = 0x7F80
    g = synth.normal_bf16(rng, (1, H), 0.1)
    rg_r, rg_y = run_rgln(res, x, g, sc, sh)
    rg_r0, rg_y0 = O.residual_gate_layernorm_modulate(res, x, g, sc, sh, EPS)
    assert_fp8_equal(run_lnq(x, sc, sh, 0.0125), O.layernorm_modulate_fp8(x, sc, sh, 0.0125, EPS),
                     "lnq non-finite")
    for got, want in ((run_ln(x, sc, sh), O.layernorm_modulate(x, sc, sh, EPS)),
                      (run_rms(x, None, sc, sh), O.rmsnorm_scale_shift(x, None, sc, sh, EPS)),
                      (rg_r, rg_r0), (rg_y, rg_y0)):
        assert_same_nans(got, want, "non-finite inputs")


@pytest.mark.parametrize("H", [1024, 3072, 4096, 3080, 520])
def test_lnq_nonfinite_modulation_and_overflowing_rows(H):
    """LN+FP8 where the output can be NaN for reasons other than the row: scale and
    shift with NaN and infinities in some columns, a scale so large that yn*(1+scale)
    overflows, rows whose squared deviations overflow, zero rows (0*inf); batch entry
    0 has finite vectors, entry 1 the bad columns, so row groups cross between them."""
    say(f"[parity] lnq non-finite modulation H={H}")
    rng = np.random.default_rng(H + 11)
    B, T = 2, 700
    x = synth.normal_bf16(rng, (B, T, H))
    big = synth.f32_to_bf16_bits(np.array([3.0e38, -3.0e38, 1.0e38], np.float32))
    for b in range(B):
        x[b, 5, : H // 2] = big[0]
        x[b, 5, H // 2:] = big[1]            # squared deviations overflow
        x[b, 9, :] = big[2]                  # constant huge row
        x[b, 13, :] = 0                      # zero row: yn = 0
        x[b, 17, 3] = 0x7F80                 # inf in a row
    sc = synth.normal_bf16(rng, (B, H), 0.1)
    sh = synth.normal_bf16(rng, (B, H), 0.1)
    cols = rng.choice(H, 12, replace=False)
    sc[1, cols[0]] = 0x7FC0                  # NaN scale
    sc[1, cols[1]] = 0x7F80                  # +inf scale (a = inf)
    sc[1, cols[2]] = 0xFF80                  # -inf scale
    sc[1, cols[3]] = synth.f32_to_bf16_bits(np.array([1.0e37], np.float32))[0]
    sh[1, cols[3]] = 0xFF80                  # p may overflow to inf, shift -inf
    sh[1, cols[4]] = 0x7FC0                  # NaN shift
    sh[1, cols[5]] = 0x7F80                  # +inf shift
    sh[1, cols[6]] = 0xFF80                  # -inf shift
    sc[1, cols[7]] = synth.f32_to_bf16_bits(np.array([3.0e38], np.float32))[0]
    for qs in (0.0125, 1.0):
        check_lnq(x, sc, sh, qs, f"lnq non-finite H={H} qscale={qs}")


@pytest.mark.parametrize("qscale", [0.0, float("inf"), float("nan"), -0.5, 1e-38, 3.0e38])
@pytest.mark.parametrize("eps", [0.0, 1e-6])
def test_lnq_special_scales_and_zero_eps(qscale, eps):
    """LN+FP8 with a quantisation scale of 0 (1/scale = inf), inf (0), NaN, negative,
    tiny or huge, and eps 0 with constant rows (a zero variance gives rstd = inf)."""
    say(f"[parity] lnq qscale={qscale} eps={eps}")
    rng = np.random.default_rng(5)
    B, T, H = 1, 40, 3072
    x = synth.normal_bf16(rng, (B, T, H))
    x[0, 3, :] = 0x3F80                      # constant row
    x[0, 4, :] = 0                           # zero row
    x[0, 5, 17] = 0x7F80                     # inf in a row
    sc = synth.normal_bf16(rng, (B, H), 0.1)
    sh = synth.normal_bf16(rng, (B, H), 0.1)
    sh[0, :8] = 0                            # y = 0 where yn = 0
    check_lnq(x, sc, sh, qscale, f"lnq qscale={qscale} eps={eps}", eps)


# --------------------------------------------------------------------------
# shapes: empty, single rows, shared vectors
# --------------------------------------------------------------------------
def test_empty_inputs():
    say("[parity] empty inputs")
    for shape in [(0, 5, 3072), (2, 0, 4096)]:
        x = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        v = torch.zeros(max(shape[0], 1), shape[2], dtype=torch.bfloat16, device="cuda")
        v = v[: shape[0]] if shape[0] else v
        y = A.adaln_layernorm_modulate(x, v, v, EPS)
        assert y.shape == x.shape


def test_single_row():
    say("[parity] single rows")
    rng = np.random.default_rng(6)
    for H in (8, 2048, 4096, 8192):
        x = synth.normal_bf16(rng, (1, 1, H))
        sc = synth.normal_bf16(rng, (1, H), 0.1)
        sh = synth.normal_bf16(rng, (1, H), 0.1)
        assert_bits_equal(run_ln(x, sc, sh), O.layernorm_modulate(x, sc, sh, EPS), f"ln H={H}")


def test_shared_vectors_batch_stride_zero():
    say("[parity] batch stride 0")
    rng = np.random.default_rng(7)
    B, T, H = 3, 11, 3072
    x = synth.normal_bf16(rng, (B, T, H))
    sc = synth.normal_bf16(rng, (1, H), 0.1)
    sh = synth.normal_bf16(rng, (1, H), 0.1)
    y = host(A.adaln_layernorm_modulate(dev(x), dev(sc), dev(sh), EPS))
    assert_bits_equal(y, O.layernorm_modulate(x, sc, sh, EPS), "bstride 0")


def test_rejected_call_leaves_outputs_untouched():
    say("[parity] rejected call")
    lib = A.load_library()
    H = 3072
    x = torch.zeros(1, 4, H, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(1, H, dtype=torch.bfloat16, device="cuda")
    y = torch.full((1, 4, H), 7.0, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    st = lib.adaln_layernorm_modulate(x.data_ptr() + 2, v.data_ptr(), v.data_ptr(), y.data_ptr(),
                                      1, 3, H, 0, 0, 1e-6, stream)
    assert st == 3  # ADALN_ERR_ALIGN
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())


# --------------------------------------------------------------------------
# batch invariance on small inputs (the large stress lives in its own file)
# --------------------------------------------------------------------------
def test_rows_alone_equal_rows_in_batch():
    say("[parity] rows alone vs in batch")
    rng = np.random.default_rng(8)
    B, T, H = 3, 17, 4096
    x = mixed_rows(rng, B, T, H)
    sc = synth.normal_bf16(rng, (B, H), 0.1)
    sh = synth.normal_bf16(rng, (B, H), 0.1)
    xd, scd, shd = dev(x), dev(sc), dev(sh)
    y = A.adaln_layernorm_modulate(xd, scd, shd, EPS)
    yr = A.adaln_rmsnorm_scale_shift(xd, None, scd, shd, EPS)
    resd = dev(mixed_rows(rng, B, T, H))
    gd = dev(synth.normal_bf16(rng, (B, H), 0.1))
    rg_r, rg_y = A.adaln_residual_gate_layernorm_modulate(resd, xd, gd, scd, shd, EPS)
    qs = torch.tensor([0.0125], dtype=torch.float32, device="cuda")
    q = A.adaln_layernorm_modulate_fp8_quant(xd, scd, shd, qs, EPS)
    for b in range(B):
        for t in range(0, T, 3):
            q1 = A.adaln_layernorm_modulate_fp8_quant(xd[b:b + 1, t:t + 1].contiguous(), scd[b],
                                                      shd[b], qs, EPS)
            assert torch.equal(q1[0, 0], q[b, t])
            r1, y1 = A.adaln_residual_gate_layernorm_modulate(
                resd[b:b + 1, t:t + 1].contiguous(), xd[b:b + 1, t:t + 1].contiguous(), gd[b],
                scd[b], shd[b], EPS)
            assert torch.equal(r1[0, 0].view(torch.int16), rg_r[b, t].view(torch.int16))
            assert torch.equal(y1[0, 0].view(torch.int16), rg_y[b, t].view(torch.int16))
            y1 = A.adaln_layernorm_modulate(xd[b:b + 1, t:t + 1].contiguous(), scd[b], shd[b], EPS)
            assert torch.equal(y1[0, 0].view(torch.int16), y[b, t].view(torch.int16))
            y2 = A.adaln_rmsnorm_scale_shift(xd[b:b + 1, t:t + 1].contiguous(), None, scd[b],
                                             shd[b], EPS)
            assert torch.equal(y2[0, 0].view(torch.int16), yr[b, t].view(torch.int16))


# --------------------------------------------------------------------------
# per-head QK RMSNorm + RoPE
# --------------------------------------------------------------------------
def check_qk(qkv, wq, wk, cs, what, eps=EPS, hk=None):
    """qkv: [tokens, 3, heads, 128] bf16 bits; q, k are its strided views."""
    T = qkv.shape[0]
    d = dev(qkv)
    q_d, k_d = d[:, 0], d[:, 1]
    q, k = qkv[:, 0], qkv[:, 1]
    if hk is not None:            # fewer K heads than Q heads
        k_d, k = k_d[:, :hk], k[:, :hk]
    qo, ko = A.adaln_qk_rmsnorm_rope(q_d, k_d, None if wq is None else dev(wq),
                                     None if wk is None else dev(wk),
                                     torch.from_numpy(cs).cuda(), eps)
    qo0, ko0 = O.qk_rmsnorm_rope(q, k, wq, wk, cs, eps)
    assert_bits_equal(host(qo), qo0, what + " q")
    assert_bits_equal(host(ko), ko0, what + " k")


def test_qk_workload_full_size():
    wl = synth.qk_rmsnorm_rope_4608x24x128()
    say(f"[parity] qk {wl.qkv.shape}")
    check_qk(wl.qkv, wl.q_weight, wl.k_weight, wl.cos_sin, "qk full size")


@pytest.mark.parametrize("T,heads", [(1, 1), (3, 2), (5, 3), (17, 5), (64, 24), (129, 48)])
def test_qk_shapes(T, heads):
    say(f"[parity] qk T={T} heads={heads}")
    rng = np.random.default_rng(T * 100 + heads)
    qkv = mixed_rows(rng, T, 3 * heads, 128).reshape(T, 3, heads, 128)
    wq = synth.normal_bf16(rng, (128,), 0.02, 1.0)
    wk = synth.normal_bf16(rng, (128,), 0.02, 1.0)
    ang = rng.uniform(-np.pi, np.pi, (T, 64))
    cs = np.concatenate([np.cos(ang), np.sin(ang)], 1).astype(np.float32)
    check_qk(qkv, wq, wk, cs, f"qk T={T} heads={heads}")
    check_qk(qkv, None, wk, cs, f"qk T={T} heads={heads} no q weight")
    if heads > 1:
        check_qk(qkv, wq, wk, cs, f"qk T={T} heads={heads} fewer k heads", hk=heads - 1)


# Q and K head counts that give one to several eight-head tasks per side, an odd
# number of tasks per token, one side absent, and token counts below and far above
# one task per resident wave (waves then step over many tokens).
@pytest.mark.parametrize("T,hq,hk", [(7, 24, 8), (600, 24, 8), (20000, 24, 8), (9000, 20, 12),
                                     (5000, 33, 1), (3000, 0, 5), (3000, 7, 0), (1, 64, 64)])
def test_qk_task_mapping(T, hq, hk):
    say(f"[parity] qk tasks T={T} hq={hq} hk={hk}")
    rng = np.random.default_rng(T + 7 * hq + hk)
    q = synth.normal_bf16(rng, (T, hq, 128))
    k = synth.normal_bf16(rng, (T, hk, 128))
    wq = synth.normal_bf16(rng, (128,), 0.02, 1.0)
    wk = synth.normal_bf16(rng, (128,), 0.02, 1.0)
    cs = synth.rope_cache(T, 128)
    qo, ko = A.adaln_qk_rmsnorm_rope(dev(q), dev(k), dev(wq), dev(wk), torch.from_numpy(cs).cuda(),
                                     EPS)
    qo0, ko0 = O.qk_rmsnorm_rope(q, k, wq, wk, cs, EPS)
    assert_bits_equal(host(qo), qo0, "q")
    assert_bits_equal(host(ko), ko0, "k")


@pytest.mark.parametrize("eps", [0.0, 1e-5, 0.25])
def test_qk_eps_and_special_rows(eps):
    say(f"[parity] qk eps={eps}")
    T, heads = 9, 4
    rng = np.random.default_rng(77)
    qkv = synth.normal_bf16(rng, (T, 3, heads, 128))
    consts = synth.f32_to_bf16_bits(np.array([0.0, -0.0, 1.0, 2.0 ** -130, 1e3, 65504.0],
                                             np.float32))
    for i, c in enumerate(consts):
        qkv[i, 0, 0, :] = c                    # constant and zero heads
    qkv[6, 1, 2, 5] = 0x7F80                   # inf
    qkv[7, 0, 3, 9] = 0x7FC0                   # nan
    cs = synth.rope_cache(T, 128)
    T_, d = qkv.shape[0], dev(qkv)
    qo, ko = A.adaln_qk_rmsnorm_rope(d[:, 0], d[:, 1], None, None, torch.from_numpy(cs).cuda(), eps)
    qo0, ko0 = O.qk_rmsnorm_rope(qkv[:, 0], qkv[:, 1], None, None, cs, eps)
    for got, want in ((host(qo), qo0), (host(ko), ko0)):
        assert_same_nans(got, want, f"qk eps={eps}")


def test_qk_heads_alone_equal_heads_in_batch():
    say("[parity] qk tokens alone vs in batch")
    rng = np.random.default_rng(5)
    T, heads = 40, 6
    qkv = synth.normal_bf16(rng, (T, 3, heads, 128))
    cs = torch.from_numpy(synth.rope_cache(T, 128)).cuda()
    d = dev(qkv)
    qo, ko = A.adaln_qk_rmsnorm_rope(d[:, 0], d[:, 1], None, None, cs, EPS)
    for t in range(0, T, 7):
        q1, k1 = A.adaln_qk_rmsnorm_rope(d[t:t + 1, 0], d[t:t + 1, 1], None, None,
                                         cs[t:t + 1].contiguous(), EPS)
        assert torch.equal(q1[0].view(torch.int16), qo[t].view(torch.int16))
        assert torch.equal(k1[0].view(torch.int16), ko[t].view(torch.int16))


# --------------------------------------------------------------------------
# residual gating on the channel-first layout
# --------------------------------------------------------------------------
def test_channel_first_full_size():
    wl = synth.rg_channel_first_2x3072x4608()
    say(f"[parity] channel-first {wl.res.shape}")
    got = A.adaln_residual_gate_channel_first(dev(wl.res), dev(wl.update), dev(wl.gate))
    assert_bits_equal(host(got), O.residual_gate_channel_first(wl.res, wl.update, wl.gate),
                      "channel-first full size")


@pytest.mark.parametrize("T", [4336, 4333, 4334, 4335])
def test_channel_first_full_size_misaligned_rows(T):
    """The token sweep's workloads at full size: rows of res/out off the 128-byte lines
    (T = 4336: 16-byte aligned; the others ragged), out of place and in place."""
    wl = synth.cf_tokens(T)
    say(f"[parity] channel-first {wl.res.shape}")
    want = O.residual_gate_channel_first(wl.res, wl.update, wl.gate)
    got = A.adaln_residual_gate_channel_first(dev(wl.res), dev(wl.update), dev(wl.gate))
    assert_bits_equal(host(got), want, f"channel-first T={T}")
    rd = dev(wl.res)
    A.adaln_residual_gate_channel_first(rd, dev(wl.update), dev(wl.gate), out=rd)
    assert_bits_equal(host(rd), want, f"channel-first T={T} in place")


@pytest.mark.parametrize("B,H,T", [(1, 8, 8), (2, 72, 40), (3, 136, 200), (1, 64, 64),
                                   (2, 3072, 72), (1, 520, 4104),
                                   # token counts with rows of res/out 8-, 4- or 2-byte aligned
                                   (2, 72, 12), (1, 136, 100), (1, 520, 4332), (2, 64, 6),
                                   (3, 8, 98), (1, 3072, 4334),
                                   (1, 8, 1), (2, 72, 7), (3, 136, 65), (2, 64, 63),
                                   (1, 520, 129), (1, 3072, 4333)])
def test_channel_first_shapes(B, H, T):
    say(f"[parity] channel-first B={B} H={H} T={T}")
    rng = np.random.default_rng(B * 7 + H + T)
    res = mixed_rows(rng, B, H, T)
    upd = mixed_rows(rng, B, T, H)
    emb = synth.normal_bf16(rng, (B, 3 * H), 0.1)
    gate = emb[:, H:2 * H]                        # a strided chunk view
    want = O.residual_gate_channel_first(res, upd, gate)
    ed = dev(emb)
    got = A.adaln_residual_gate_channel_first(dev(res), dev(upd), ed[:, H:2 * H])
    assert_bits_equal(host(got), want, f"cf B={B} H={H} T={T}")
    # in place on the residual
    rd = dev(res)
    A.adaln_residual_gate_channel_first(rd, dev(upd), ed[:, H:2 * H], out=rd)
    assert_bits_equal(host(rd), want, f"cf in place B={B} H={H} T={T}")
    # one gate vector for the batch
    g1 = synth.normal_bf16(rng, (1, H), 0.1)
    got = A.adaln_residual_gate_channel_first(dev(res), dev(upd), dev(g1))
    assert_bits_equal(host(got), O.residual_gate_channel_first(res, upd, g1), "cf shared gate")


# --------------------------------------------------------------------------
# the FP8 kernel's quantisation step, exhaustively over binary32
# --------------------------------------------------------------------------
def test_device_fp8_quant_all_fp32_patterns():
    # qscale 1: the clamp and the E4M3 conversion of every fp32 pattern, against
    # torch's float8_e4m3fn conversion of the clamped value (the eager chain)
    qs = torch.ones(1, dtype=torch.float32, device="cuda")
    n_chunks = 16
    step = (1 << 32) // n_chunks
    for k in range(n_chunks):
        say(f"[diag] fp8 quant chunk {k + 1}/{n_chunks}")
        u = torch.arange(k * step, (k + 1) * step, dtype=torch.int64, device="cuda")
        f = (u - (1 << 32) * (u >= (1 << 31)).long()).to(torch.int32).view(torch.float32)
        got = A.adaln_diag_quant_fp8(f, qs)
        want = f.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
        gn = (got & 0x7F) == 0x7F
        wn = (want & 0x7F) == 0x7F
        assert torch.equal(gn, wn), f"chunk {k}: NaN positions"
        assert torch.equal(got[~gn], want[~wn]), f"chunk {k}"
        assert bool((got[gn] == 0xFF).all()), f"chunk {k}: a NaN code other than 0xFF"
        del u, f, got, want, gn, wn
    torch.cuda.synchronize()


@pytest.mark.parametrize("qscale", [0.0125, 3.0, 2.0 ** -20, 1e30])
def test_device_fp8_quant_scaled_vs_oracle(qscale):
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    qs = torch.tensor([qscale], dtype=torch.float32, device="cuda")
    got = A.adaln_diag_quant_fp8(torch.from_numpy(v.copy()).cuda(), qs).cpu().numpy()
    inv = np.float32(1.0) / np.float32(qscale)
    with np.errstate(over="ignore", invalid="ignore"):
        t = np.clip(v * inv, np.float32(-448.0), np.float32(448.0))
    assert_fp8_equal(got, O.to_e4m3fn(t), f"quant qscale={qscale}")


# --------------------------------------------------------------------------
# the streaming copy used as the bench's ceiling
# --------------------------------------------------------------------------
def test_stream_copy_is_exact():
    say("[diag] stream copy")
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    for n16 in (1, 255, 2048, 2049, 123457, 4216 * 512):
        src = torch.randint(-(1 << 31), (1 << 31) - 1, (n16 * 4,), dtype=torch.int32,
                            device="cuda", generator=g)
        full = torch.full((n16 * 4 + 64,), 7, dtype=torch.int32, device="cuda")
        dst = full[: n16 * 4]
        A.adaln_diag_stream_copy(src, dst)
        assert torch.equal(src, dst), n16
        assert bool((full[n16 * 4:] == 7).all()), "wrote past the end"
    lib = A.load_library()
    assert lib.adaln_diag_stream_copy(None, None, 0, None) == 0
    assert lib.adaln_diag_stream_copy(src.data_ptr(), dst.data_ptr(), 24, None) == 2  # SHAPE
    assert lib.adaln_diag_stream_copy(src.data_ptr(), src.data_ptr() + 16, 64, None) == 5


@pytest.mark.parametrize("per", [1, 2, 4, 8, 16])
def test_stream_kernels_do_what_they_say(per):
    """The measured ceilings come from these kernels: the copy copies, the fill fills,
    and the read folds every loaded word (its output is the XOR fold of the data of
    each wave: 64 lanes x per vectors of 16 bytes, a wave covering 1024*per bytes in
    the order the grid assigns them)."""
    say(f"[diag] stream kernels per={per}")
    g = torch.Generator(device="cuda")
    g.manual_seed(per)
    for n16 in (1, 255, 4096 * per + 17, 50000):
        src = torch.randint(-(1 << 31), (1 << 31) - 1, (n16 * 4,), dtype=torch.int32,
                            device="cuda", generator=g)
        full = torch.full((n16 * 4 + 64,), 7, dtype=torch.int32, device="cuda")
        dst = full[: n16 * 4]
        A.adaln_diag_stream("copy", src, dst, per)
        assert torch.equal(src, dst) and bool((full[n16 * 4:] == 7).all()), ("copy", n16)
        full.fill_(7)
        A.adaln_diag_stream("fill", None, dst, per)
        assert bool((full[n16 * 4:] == 7).all()), ("fill past the end", n16)
        pat = torch.tensor([0x3F803F80, 0x3F803F80 ^ 0x9E3779B9], dtype=torch.int64)
        pat = ((pat + (1 << 31)) % (1 << 32) - (1 << 31)).to(torch.int32).cuda()
        assert torch.equal(dst.view(-1, 2), pat.expand(n16 * 2, 2)), ("fill", n16)
        full.fill_(7)
        A.adaln_diag_stream("read", src, dst, per)
        # expected folds: thread t of workgroup b reads vectors b*256*per + k*256 + t
        v = src.view(-1, 4).cpu().numpy().astype(np.uint32)
        words = np.bitwise_xor.reduce(v, axis=1)
        blocks = -(-n16 // (256 * per))
        pad = np.zeros(blocks * 256 * per, np.uint32)
        pad[:n16] = words
        per_thread = np.bitwise_xor.reduce(pad.reshape(blocks, per, 256), axis=1)
        want = np.bitwise_xor.reduce(per_thread.reshape(blocks, 4, 64), axis=2).reshape(-1)
        got = dst[: blocks * 4].cpu().numpy().astype(np.uint32)
        assert np.array_equal(got, want), ("read", n16)
        assert bool((dst[blocks * 4:] == 7).all()), ("read wrote past its folds", n16)


# --------------------------------------------------------------------------
# the device's rounding and finalize steps, exhaustively
# --------------------------------------------------------------------------
def test_device_bf16_rounding_all_fp32_patterns():
    # torch's float32 -> bfloat16 conversion (nearest-even) is the reference; NaN
    # inputs must stay NaN.
    n_chunks = 16
    step = (1 << 32) // n_chunks
    for k in range(n_chunks):
        say(f"[diag] bf16 rounding chunk {k + 1}/{n_chunks}")
        u = torch.arange(k * step, (k + 1) * step, dtype=torch.int64, device="cuda")
        f = (u - (1 << 32) * (u >= (1 << 31)).long()).to(torch.int32).view(torch.float32)
        got = A.adaln_diag_round_bf16(f).view(torch.int16)
        want = f.to(torch.bfloat16).view(torch.int16)
        nan = torch.isnan(f)
        assert torch.equal(got[~nan], want[~nan]), f"chunk {k}"
        gw = got[nan].to(torch.int32) & 0xFFFF
        assert bool(((gw & 0x7F80) == 0x7F80).all() and ((gw & 0x7F) != 0).all())
        # a quiet NaN with the input's sign (the oracle writes 0x7FC0 | sign; the
        # payload of a NaN is not part of the numerics, its sign and quietness are)
        sign_in = (u[nan] >> 31).to(torch.int32)
        assert bool(((gw >> 15) == sign_in).all()), f"chunk {k}: NaN sign"
        assert bool(((gw & 0x0040) != 0).all()), f"chunk {k}: NaN not quiet"
        del u, f, got, want, nan, gw, sign_in
    torch.cuda.synchronize()


@pytest.mark.parametrize("H,eps", [(1, 1e-6), (3072, 1e-6), (8168, 0.0), (520, 1e-5)])
def test_device_finalize_all_nonnegative_stats(H, eps):
    # stat S in [+0, +inf] over H elements: rstd = RN(1/RN(sqrt(RN(RN(S/H) + eps)))),
    # by the kernels' own code, shortcuts included (waves with every lane in range
    # take them; 3072 = 3 * 2^10, 8168 = 8 * 1021 and 520 = 8 * 65 are not powers of
    # two; eps 0 reaches the smallest roots).  Reference: divide, sqrt and reciprocal
    # in float64 rounded once to float32 (a double rounding through binary64 equals
    # the single fp32 rounding for divide and sqrt, since 53 >= 2*24 + 2), the add
    # in fp32.
    e = torch.tensor(eps, dtype=torch.float32, device="cuda")
    top = 0x7F800000 + 1
    n_chunks = 16
    step = (top + n_chunks - 1) // n_chunks
    for k in range(n_chunks):
        say(f"[diag] finalize H={H} eps={eps} chunk {k + 1}/{n_chunks}")
        lo, hi = k * step, min(top, (k + 1) * step)
        s = torch.arange(lo, hi, dtype=torch.int32, device="cuda").view(torch.float32)
        got = A.adaln_diag_finalize(s, eps, H=H)
        v = (s.double() / H).float() + e
        root = v.double().sqrt().float()
        want = (1.0 / root.double()).float()
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), f"chunk {k}"
        del s, got, v, root, want
    # host IEEE arithmetic on a sample, independent of torch's device math
    rng = np.random.default_rng(H)
    bits = rng.integers(0, 0x7F800000, size=1 << 22, dtype=np.uint32)
    s = bits.view(np.float32)
    got = A.adaln_diag_finalize(torch.from_numpy(s.copy()).cuda(), eps, H=H).cpu().numpy()
    v = (s.astype(np.float64) / H).astype(np.float32) + np.float32(eps)
    with np.errstate(divide="ignore"):  # 1/sqrt(+0) is +inf, as on the device
        want = np.float32(1.0) / np.sqrt(v)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_binding_rejects_wrong_outputs():
    """Outputs of the wrong shape, or outside the inputs' device, are refused before
    any launch (the library cannot see a buffer's size)."""
    say("[parity] binding output checks")
    x = torch.zeros((1, 4, 64), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((1, 64), dtype=torch.bfloat16, device="cuda")
    small = torch.empty((1, 3, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="shape"):
        A.adaln_layernorm_modulate(x, v, v, out=small)
    with pytest.raises(ValueError, match="shape"):
        A.adaln_residual_gate_layernorm_modulate(x, x, v, v, v, r_out=small)
    with pytest.raises(ValueError):
        A.adaln_layernorm_modulate(x, v, v, out=torch.empty((1, 4, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        A.adaln_layernorm_modulate(x, v.cpu(), v)
    q = torch.zeros((2, 3, 128), dtype=torch.bfloat16, device="cuda")
    cs = torch.zeros((2, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="shape"):
        A.adaln_qk_rmsnorm_rope(q, q, None, None, cs,
                                q_out=torch.empty((2, 2, 128), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
