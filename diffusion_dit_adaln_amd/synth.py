"""Seeded synthetic inputs for the fused adaLN normalisation path.

This module only draws random numbers and stores them as bfloat16 bit patterns
(numpy ``uint16``).  It holds none of the method's arithmetic; the library and the
CPU oracle both take their inputs from here.

Recipe (shared by tests, the smoke check and the benchmark):
  * every tensor has its own numpy ``PCG64`` stream seeded by
    ``SeedSequence([seed, stream, tensor_id])`` (a stream number per workload);
  * values are drawn as float64 standard normals, multiplied by sigma (a standard
    deviation) and offset by mu in float64, cast to float32, then rounded to
    bfloat16 (nearest-even) by torch's dtype conversion;
  * outliers: ``round(frac * N)`` positions chosen without replacement are
    multiplied by the factor in float32 before the bf16 rounding.

Workload shapes follow the pages: the FLUX.1 adaLN site shapes (PR #34126 report,
test snippet: hidden 3072, 4096 image + 512 text tokens, a CFG batch of 2), the
ERNIE-Image shapes (PR #33854 report, tests: (1,4216,4096), (2,1140,4096),
(1,128,2048)) and the contract docstring shapes in the sglang diffusion kernels
guide (add-a-kernel workflow, step 4).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

TENSOR_IDS = {"x": 0, "scale": 1, "shift": 2, "gate": 3, "res": 4, "weight": 5, "mask": 6,
              "tokens": 7, "class": 8}


def _rng(seed: int, stream: int, tensor: str) -> np.random.Generator:
    """The generator of one tensor of one workload: stream numbers keep the workloads'
    draws apart."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [seed, stream, TENSOR_IDS[tensor]])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns via torch's conversion (nearest-even)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    t = torch.from_numpy(a).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, sigma: float = 1.0, mu: float = 0.0,
                outlier_frac: float = 0.0, outlier_factor: float = 1.0,
                chunk: int = 1 << 24) -> np.ndarray:
    """bf16 bits of mu + sigma*N(0,1), drawn in float64, optional outliers."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, np.uint16)
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        v = rng.standard_normal(hi - lo) * sigma + mu
        out[lo:hi] = f32_to_bf16_bits(v.astype(np.float32))
    if outlier_frac > 0.0:
        k = int(round(outlier_frac * n))
        pos = rng.choice(n, size=k, replace=False)
        v = bf16_bits_to_f32(out[pos]) * np.float32(outlier_factor)
        out[pos] = f32_to_bf16_bits(v)
    return out.reshape(shape)


@dataclasses.dataclass
class Workload:
    """One synthetic invocation of an entry point (arrays are bf16 bits)."""
    op: str                      # "ln" | "rms" | "rg" | "rgln" | "lnq"
    name: str
    x: np.ndarray                # [B,T,H]
    scale: np.ndarray            # [B,H] (possibly a strided view)
    shift: np.ndarray            # [B,H]
    weight: np.ndarray | None = None  # [H] (rms / rg)
    gate: np.ndarray | None = None    # [B,H] (rg, rgln)
    res: np.ndarray | None = None     # [B,T,H] (rg, rgln)
    eps: float = 1e-6
    qscale: float | None = None       # lnq: static FP8 quantisation scale

    @property
    def shape(self):
        return self.x.shape

    def algorithmic_bytes(self) -> int:
        """HBM bytes the path must move: read x[,res], write y[,r] (bf16)."""
        n = int(np.prod(self.x.shape))
        if self.op == "lnq":
            return 3 * n  # read x (bf16), write q (one byte)
        return (8 if self.op in ("rg", "rgln") else 4) * n


def _vecs(seed, stream, B, H, names, sigma=0.1):
    return {n: normal_bf16(_rng(seed, stream, n), (B, H), sigma) for n in names}


def ln_1x128x2048(seed: int = 0) -> Workload:
    """LayerNorm (no affine, eps 1e-6) + modulate, x [1,128,2048] ~ N(0,1),
    scale/shift [1,2048] ~ 0.1*N(0,1)."""
    B, T, H = 1, 128, 2048
    v = _vecs(seed, 0, B, H, ["scale", "shift"])
    return Workload("ln", "ln_1x128x2048", normal_bf16(_rng(seed, 0, "x"), (B, T, H)),
                    v["scale"], v["shift"])


def rms_1x4216x4096(seed: int = 0) -> Workload:
    """RMSNorm (weight 1+0.02*N, eps 1e-6) + scale/shift, x [1,4216,4096] ~ N(0,1)
    with 0.1% of entries multiplied by 50; scale/shift [1,4096] ~ 0.1*N."""
    B, T, H = 1, 4216, 4096
    v = _vecs(seed, 1, B, H, ["scale", "shift"])
    w = normal_bf16(_rng(seed, 1, "weight"), (H,), 0.02, 1.0)
    x = normal_bf16(_rng(seed, 1, "x"), (B, T, H), outlier_frac=0.001, outlier_factor=50.0)
    return Workload("rms", "rms_1x4216x4096", x, v["scale"], v["shift"], weight=w)


def rms_rows(T: int, seed: int = 0) -> Workload:
    """The headline RMS workload's distributions with T rows of H = 4096 (for size
    sweeps): x [1,T,4096] ~ N(0,1) with 0.1% of entries multiplied by 50."""
    B, H = 1, 4096
    v = _vecs(seed, 1, B, H, ["scale", "shift"])
    w = normal_bf16(_rng(seed, 1, "weight"), (H,), 0.02, 1.0)
    x = normal_bf16(_rng(seed, 1, "x"), (B, T, H), outlier_frac=0.001, outlier_factor=50.0)
    return Workload("rms", f"rms_1x{T}x4096", x, v["scale"], v["shift"], weight=w)


def ln_rows(T: int, seed: int = 0) -> Workload:
    """LayerNorm (no affine, eps 1e-6) + modulate with T rows of H = 3072 (the FLUX.1
    site width, for size sweeps): x [1,T,3072] ~ N(0,1), scale/shift ~ 0.1*N."""
    B, H = 1, 3072
    v = _vecs(seed, 2, B, H, ["scale", "shift"])
    return Workload("ln", f"ln_1x{T}x3072", normal_bf16(_rng(seed, 2, "x"), (B, T, H)),
                    v["scale"], v["shift"])


def rg_rms_2x1140x4096(seed: int = 0) -> Workload:
    """Residual-gate RMSNorm + scale/shift (CFG batch): res, x [2,1140,4096] ~ N(0,1);
    gate/scale/shift [2,4096] ~ 0.1*N; no weight."""
    B, T, H = 2, 1140, 4096
    v = _vecs(seed, 2, B, H, ["scale", "shift", "gate"])
    return Workload("rg", "rg_rms_2x1140x4096", normal_bf16(_rng(seed, 2, "x"), (B, T, H)),
                    v["scale"], v["shift"], weight=None, gate=v["gate"],
                    res=normal_bf16(_rng(seed, 2, "res"), (B, T, H)))


def _flux_ln(seed, B, T, H, stream):
    v = _vecs(seed, stream, B, H, ["scale", "shift"])
    return Workload("ln", f"ln_{B}x{T}x{H}", normal_bf16(_rng(seed, stream, "x"), (B, T, H)),
                    v["scale"], v["shift"])


def ln_2x4608x3072(seed: int = 0) -> Workload:
    """FLUX.1-like LayerNorm + modulate: x [2,4608,3072] (4096 image + 512 text
    tokens, CFG batch) ~ N(0,1); scale/shift [2,3072] ~ 0.1*N."""
    return _flux_ln(seed, 2, 4608, 3072, 3)


def ln_1x4333x3072(seed: int = 0) -> Workload:
    """FLUX.1-like LayerNorm + modulate at a ragged token count: x [1,4333,3072] ~
    N(0,1); scale/shift [1,3072] ~ 0.1*N."""
    return _flux_ln(seed, 1, 4333, 3072, 33)


def rg_ln_2x4096x3072(seed: int = 0) -> Workload:
    """Residual-gate LayerNorm + modulate at the FLUX.1 dual-stream image-token site
    (hidden 3072, 4096 image tokens, CFG batch of 2): res, x [2,4096,3072] ~ N(0,1);
    gate/scale/shift [2,3072] ~ 0.1*N."""
    B, T, H = 2, 4096, 3072
    v = _vecs(seed, 5, B, H, ["scale", "shift", "gate"])
    return Workload("rgln", "rg_ln_2x4096x3072", normal_bf16(_rng(seed, 5, "x"), (B, T, H)),
                    v["scale"], v["shift"], gate=v["gate"],
                    res=normal_bf16(_rng(seed, 5, "res"), (B, T, H)))


def ln_fp8_2x4608x3072(seed: int = 0) -> Workload:
    """LayerNorm + modulate + static FP8 quantisation at the FLUX site shape
    x [2,4608,3072] ~ N(0,1); scale/shift [2,3072] ~ 0.1*N; static scale 0.0125
    (about amax/448 of the modulated activations)."""
    B, T, H = 2, 4608, 3072
    v = _vecs(seed, 6, B, H, ["scale", "shift"])
    return Workload("lnq", "ln_fp8_2x4608x3072", normal_bf16(_rng(seed, 6, "x"), (B, T, H)),
                    v["scale"], v["shift"], qscale=0.0125)


def rope_cache(tokens: int, head_dim: int, base: float = 10000.0) -> np.ndarray:
    """float32 [tokens, head_dim]: row t = cos(t*theta_i) for i < head_dim/2, then
    sin(t*theta_i), theta_i = base^(-2i/head_dim); angles and cos/sin in float64, then
    cast to float32.  (An input of the QK-norm + RoPE op, like the cos/sin cache a
    model precomputes.)"""
    i = np.arange(head_dim // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / head_dim)
    ang = np.arange(tokens, dtype=np.float64)[:, None] * theta[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


@dataclasses.dataclass
class QKWorkload:
    """Per-head QK RMSNorm + RoPE input: q, k are views of one packed QKV buffer."""
    name: str
    qkv: np.ndarray          # [tokens, 3, heads, head_dim] bf16 bits (q, k, v)
    q_weight: np.ndarray     # [head_dim]
    k_weight: np.ndarray     # [head_dim]
    cos_sin: np.ndarray      # float32 [tokens, head_dim]
    eps: float = 1e-6
    op: str = "qk"

    @property
    def q(self):
        return self.qkv[:, 0]

    @property
    def k(self):
        return self.qkv[:, 1]

    def algorithmic_bytes(self) -> int:
        """Read q and k, write q_out and k_out (bf16), read the cos/sin cache once."""
        T, _, Hd, D = self.qkv.shape
        return 8 * T * Hd * D + 4 * T * D


def qk_rmsnorm_rope_4608x24x128(seed: int = 0) -> QKWorkload:
    """Qwen-Image-like attention input (Qwen PR report: batch 1, head_dim 128, Q/K as
    views of the packed QKV projection): 4096 image + 512 text tokens, 24 heads of 128
    (hidden 3072); qkv ~ N(0,1); RMSNorm weights 1 + 0.02*N; RoPE cache of positions
    0..4607 with base 10000."""
    T, Hd, D = 4608, 24, 128
    qkv = normal_bf16(_rng(seed, 7, "x"), (T, 3, Hd, D))
    return QKWorkload("qk_rmsnorm_rope_4608x24x128", qkv,
                      normal_bf16(_rng(seed, 7, "weight"), (D,), 0.02, 1.0),
                      normal_bf16(_rng(seed, 7, "scale"), (D,), 0.02, 1.0),
                      rope_cache(T, D))


@dataclasses.dataclass
class CFWorkload:
    """Residual gating on a channel-first residual: res [B,H,T], update [B,T,H]."""
    name: str
    res: np.ndarray          # [B, H, T] bf16 bits
    update: np.ndarray       # [B, T, H]
    gate: np.ndarray         # [B, H]
    op: str = "cf"

    def algorithmic_bytes(self) -> int:
        """Read res and update, write out (bf16)."""
        return 6 * int(np.prod(self.res.shape))


def rg_channel_first_2x3072x4608(seed: int = 0) -> CFWorkload:
    """Channel-first residual gating at the FLUX site size: hidden 3072, 4608 tokens,
    CFG batch 2; res, update ~ N(0,1); gate ~ 0.1*N."""
    B, H, T = 2, 3072, 4608
    return CFWorkload("rg_channel_first_2x3072x4608",
                      normal_bf16(_rng(seed, 8, "res"), (B, H, T)),
                      normal_bf16(_rng(seed, 8, "x"), (B, T, H)),
                      normal_bf16(_rng(seed, 8, "gate"), (B, H), 0.1))


def cf_tokens(T: int, seed: int = 0) -> CFWorkload:
    """Channel-first residual gating at hidden 3072, CFG batch 2, with T tokens (the
    token-count sweep: T % 8 decides whether the residual rows are 16-byte aligned, and
    T % 64 whether they start on 128-byte lines)."""
    B, H = 2, 3072
    return CFWorkload(f"rg_channel_first_2x3072x{T}",
                      normal_bf16(_rng(seed, 38, "res"), (B, H, T)),
                      normal_bf16(_rng(seed, 38, "x"), (B, T, H)),
                      normal_bf16(_rng(seed, 38, "gate"), (B, H), 0.1))


def flux_chunk_views(seed: int, B: int, H: int, chunks: int, stream: int = 30):
    """scale/shift as strided views of one [B, chunks*H] embedding, like
    ``emb.chunk(chunks, dim=1)`` in the FLUX.1 test snippet: (emb, shift, scale)
    with shift = part 0 and scale = part 1, batch stride chunks*H."""
    emb = normal_bf16(_rng(seed, stream, "scale"), (B, chunks * H), 1.0)
    return emb, emb[:, 0:H], emb[:, H:2 * H]


@dataclasses.dataclass
class StressSets:
    """Batch-invariance stress workload: packed row-sets of one hidden size."""
    x: np.ndarray            # [R, H] all sets' rows, packed
    offsets: np.ndarray      # [S+1] row offsets of the sets
    row_class: np.ndarray    # [R] 0: N(0,1), 1: 1e-3*N(0,1), 2: 1e3*N(0,1)
    scale: np.ndarray        # [S, H] per-set modulation
    shift: np.ndarray        # [S, H]
    weight: np.ndarray       # [H] (RMSNorm variant), 1 + 0.02*N


CLASS_SIGMA = (1.0, 1e-3, 1e3)


def ragged_sets(seed: int = 0, n_sets: int = 256, max_tokens: int = 4096, H: int = 3072,
                stream: int = 4) -> StressSets:
    """256 packed row-sets, token counts uniform in [1, max_tokens], hidden 3072;
    each row is N(0,1), 1e-3*N(0,1) or 1e3*N(0,1) with equal probability."""
    tr = _rng(seed, stream, "tokens")
    counts = tr.integers(1, max_tokens + 1, size=n_sets)
    offsets = np.zeros(n_sets + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    R = int(offsets[-1])
    cls = _rng(seed, stream, "class").integers(0, 3, size=R).astype(np.int8)
    xr = _rng(seed, stream, "x")
    x = np.empty((R, H), np.uint16)
    step = max(1, (1 << 22) // H)
    sig = np.array(CLASS_SIGMA, np.float64)
    for lo in range(0, R, step):
        hi = min(R, lo + step)
        v = xr.standard_normal((hi - lo, H)) * sig[cls[lo:hi]][:, None]
        x[lo:hi] = f32_to_bf16_bits(v.astype(np.float32))
    v = _vecs(seed, stream, n_sets, H, ["scale", "shift"])
    w = normal_bf16(_rng(seed, stream, "weight"), (H,), 0.02, 1.0)
    return StressSets(x, offsets, cls, v["scale"], v["shift"], w)


@dataclasses.dataclass
class StressSetsDevice:
    """The batch-invariance stress workload drawn on the device (torch tensors)."""
    x: "torch.Tensor"        # [R, H] bfloat16, packed row-sets
    offsets: np.ndarray      # [S+1] row offsets
    row_class: np.ndarray    # [R] 0: N(0,1), 1: 1e-3*N(0,1), 2: 1e3*N(0,1)
    scale: "torch.Tensor"    # [S, H] bfloat16
    shift: "torch.Tensor"    # [S, H] bfloat16
    weight: "torch.Tensor"   # [H] bfloat16, 1 + 0.02*N


def ragged_sets_device(seed: int = 0, n_sets: int = 256, max_tokens: int = 4096, H: int = 3072,
                       device: str = "cuda", stream: int = 4) -> StressSetsDevice:
    """Same recipe as ragged_sets (set sizes and row classes from the numpy streams),
    but the ~1.6e9 activations are drawn on the device with torch's seeded
    generator: float32 N(0,1) times the row's sigma, rounded to bfloat16."""
    tr = _rng(seed, stream, "tokens")
    counts = tr.integers(1, max_tokens + 1, size=n_sets)
    offsets = np.zeros(n_sets + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    R = int(offsets[-1])
    cls = _rng(seed, stream, "class").integers(0, 3, size=R).astype(np.int8)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(np.random.SeedSequence([seed, stream, TENSOR_IDS["x"]]).generate_state(1)[0]))
    sig = torch.tensor(CLASS_SIGMA, dtype=torch.float32, device=device)[
        torch.from_numpy(cls.astype(np.int64)).to(device)]
    x = torch.empty((R, H), dtype=torch.bfloat16, device=device)
    step = 1 << 16
    for lo in range(0, R, step):
        hi = min(R, lo + step)
        v = torch.randn((hi - lo, H), generator=gen, device=device, dtype=torch.float32)
        x[lo:hi] = (v * sig[lo:hi, None]).to(torch.bfloat16)
    v = _vecs(seed, stream, n_sets, H, ["scale", "shift"])
    w = normal_bf16(_rng(seed, stream, "weight"), (H,), 0.02, 1.0)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

    return StressSetsDevice(x, offsets, cls, to_dev(v["scale"]), to_dev(v["shift"]), to_dev(w))


def ragged_residual_device(st: StressSetsDevice, seed: int = 0, stream: int = 4,
                           device: str = "cuda"):
    """The residual stream and per-set gates for the gated ops on the stress sets:
    res [R, H] bfloat16 N(0,1) drawn on the device with its own seeded generator,
    gate [S, H] bfloat16 0.1*N(0,1)."""
    R, H = st.x.shape
    S = len(st.offsets) - 1
    gen = torch.Generator(device=device)
    gen.manual_seed(int(np.random.SeedSequence([seed, stream, TENSOR_IDS["res"]])
                        .generate_state(1)[0]))
    res = torch.empty((R, H), dtype=torch.bfloat16, device=device)
    step = 1 << 16
    for lo in range(0, R, step):
        hi = min(R, lo + step)
        res[lo:hi] = torch.randn((hi - lo, H), generator=gen, device=device,
                                 dtype=torch.float32).to(torch.bfloat16)
    g = _vecs(seed, stream, S, H, ["gate"])["gate"]
    gate = torch.from_numpy(np.ascontiguousarray(g).view(np.int16)).view(torch.bfloat16).to(device)
    return res, gate


# the benchmark and parity workloads by name (bench.py --workload NAME)
WORKLOADS = {
    "ln_1x128x2048": ln_1x128x2048,
    "rms_1x4216x4096": rms_1x4216x4096,
    "rg_rms_2x1140x4096": rg_rms_2x1140x4096,
    "ln_2x4608x3072": ln_2x4608x3072,
    "ln_1x4333x3072": ln_1x4333x3072,
    "rg_ln_2x4096x3072": rg_ln_2x4096x3072,
    "ln_fp8_2x4608x3072": ln_fp8_2x4608x3072,
    "qk_rmsnorm_rope_4608x24x128": qk_rmsnorm_rope_4608x24x128,
    "rg_channel_first_2x3072x4608": rg_channel_first_2x3072x4608,
}
