"""ctypes wrapper around the C oracle (``adaln_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path (the HIP library and its
binding) never imports this module.

Arrays are numpy ``uint16`` holding raw bfloat16 bit patterns.  Per-batch vectors
may be strided 2-D views ``[B, H]`` (for example slices of a larger embedding, as
``emb.chunk(k, dim=1)`` produces); their inner stride must be one element.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "adaln_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

# binary32 evaluated exactly as written: no contraction to FMA, no fast-math,
# SSE arithmetic (FLT_EVAL_METHOD 0).
GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
             "-fexcess-precision=standard", "-msse2", "-mfpmath=sse", "-Wall", "-Wextra"]

STATS_PER_ROW = 6

_lib = None


def build() -> None:
    """Compile the oracle (always; cheap)."""
    tmp = LIB + ".tmp"
    subprocess.check_call(["gcc", *GCC_FLAGS, SRC, "-o", tmp, "-lm"])
    os.replace(tmp, LIB)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    lib = ctypes.CDLL(LIB)
    P = ctypes.c_void_p
    I = ctypes.c_int64
    F = ctypes.c_float
    lib.oracle_layout.argtypes = [I, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                  ctypes.POINTER(ctypes.c_int)]
    lib.oracle_layout.restype = ctypes.c_int
    lib.oracle_layernorm_modulate.argtypes = [P, P, P, P, I, I, I, I, I, F, P, P]
    lib.oracle_layernorm_modulate.restype = ctypes.c_int
    lib.oracle_rmsnorm_scale_shift.argtypes = [P, P, P, P, P, I, I, I, I, I, F, P, P]
    lib.oracle_rmsnorm_scale_shift.restype = ctypes.c_int
    lib.oracle_residual_gate_rmsnorm_scale_shift.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I,
                                                             I, F, P, P]
    lib.oracle_residual_gate_rmsnorm_scale_shift.restype = ctypes.c_int
    lib.oracle_residual_gate_layernorm_modulate.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I,
                                                            F, P, P]
    lib.oracle_residual_gate_layernorm_modulate.restype = ctypes.c_int
    lib.oracle_layernorm_modulate_fp8.argtypes = [P, P, P, F, P, I, I, I, I, I, F, P, P]
    lib.oracle_layernorm_modulate_fp8.restype = ctypes.c_int
    lib.oracle_to_e4m3fn.argtypes = [P, P, I]
    lib.oracle_to_e4m3fn.restype = None
    lib.oracle_quant_fp8.argtypes = [P, P, I, F]
    lib.oracle_quant_fp8.restype = None
    lib.oracle_qk_rmsnorm_rope.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, F, P, P]
    lib.oracle_qk_rmsnorm_rope.restype = ctypes.c_int
    lib.oracle_residual_gate_channel_first.argtypes = [P, P, P, P, I, I, I, I]
    lib.oracle_residual_gate_channel_first.restype = ctypes.c_int
    lib.oracle_round_bf16.argtypes = [P, P, I]
    lib.oracle_round_bf16.restype = None
    lib.oracle_modulate.argtypes = [P, P, P, P, I]
    lib.oracle_modulate.restype = None
    lib.oracle_gate_residual.argtypes = [P, P, P, P, I]
    lib.oracle_gate_residual.restype = None
    assert lib.oracle_stats_per_row() == STATS_PER_ROW
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _act(a, name):
    a = np.asarray(a)
    if a.dtype != np.uint16 or a.ndim != 3 or not a.flags.c_contiguous:
        raise ValueError(f"{name}: expected a C-contiguous uint16 [B,T,H] array")
    return a


def _vec(v, B, H, name):
    """Return (view, batch stride in elements) for a per-batch vector argument."""
    v = np.asarray(v)
    if v.dtype != np.uint16:
        raise ValueError(f"{name}: expected uint16 bf16 bits")
    if v.ndim == 1:
        v = v.reshape(1, -1)
    if v.ndim != 2 or v.shape[1] != H or v.strides[1] != 2 or v.shape[0] not in (1, B):
        raise ValueError(f"{name}: expected [B,H] or [1,H] with unit inner stride, got {v.shape}")
    bstride = v.strides[0] // 2 if v.shape[0] == B and B > 1 else 0
    return v, bstride


def layout(H: int):
    """(waves per row, lanes per row, chunks per lane) of the fixed order for H."""
    lib = _load()
    w, p, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    if lib.oracle_layout(H, ctypes.byref(w), ctypes.byref(p), ctypes.byref(c)) != 0:
        raise ValueError(f"unsupported H={H}")
    return w.value, p.value, c.value


def _check(rc, what):
    if rc < 0:
        raise ValueError(f"{what}: rejected arguments")
    if rc > 0:
        raise AssertionError(f"{what}: lanes disagreed after the butterfly on {rc} rows")


def layernorm_modulate(x, scale, shift, eps=1e-6, want_norm=False, want_stats=False):
    lib = _load()
    x = _act(x, "x")
    B, T, H = x.shape
    sc, sbs = _vec(scale, B, H, "scale")
    sh, hbs = _vec(shift, B, H, "shift")
    y = np.empty_like(x)
    yn = np.empty_like(x) if want_norm else None
    st = np.empty((B * T, STATS_PER_ROW), np.float32) if want_stats else None
    rc = lib.oracle_layernorm_modulate(_ptr(x), _ptr(sc), _ptr(sh), _ptr(y), B, T, H, sbs, hbs,
                                       float(np.float32(eps)), _ptr(yn), _ptr(st))
    _check(rc, "layernorm_modulate")
    return _ret(y, yn, st, want_norm, want_stats)


def rmsnorm_scale_shift(x, weight, scale, shift, eps=1e-6, want_norm=False, want_stats=False):
    lib = _load()
    x = _act(x, "x")
    B, T, H = x.shape
    if weight is not None:
        weight = np.ascontiguousarray(weight, dtype=np.uint16).reshape(H)
    sc, sbs = _vec(scale, B, H, "scale")
    sh, hbs = _vec(shift, B, H, "shift")
    y = np.empty_like(x)
    yn = np.empty_like(x) if want_norm else None
    st = np.empty((B * T, STATS_PER_ROW), np.float32) if want_stats else None
    rc = lib.oracle_rmsnorm_scale_shift(_ptr(x), _ptr(weight), _ptr(sc), _ptr(sh), _ptr(y), B, T, H,
                                        sbs, hbs, float(np.float32(eps)), _ptr(yn), _ptr(st))
    _check(rc, "rmsnorm_scale_shift")
    return _ret(y, yn, st, want_norm, want_stats)


def residual_gate_rmsnorm_scale_shift(res, x, gate, weight, scale, shift, eps=1e-6,
                                      want_norm=False, want_stats=False):
    """Returns (r, y[, yn][, stats])."""
    lib = _load()
    res = _act(res, "res")
    x = _act(x, "x")
    if res.shape != x.shape:
        raise ValueError("res and x shapes differ")
    B, T, H = x.shape
    if weight is not None:
        weight = np.ascontiguousarray(weight, dtype=np.uint16).reshape(H)
    g, gbs = _vec(gate, B, H, "gate")
    sc, sbs = _vec(scale, B, H, "scale")
    sh, hbs = _vec(shift, B, H, "shift")
    r = np.empty_like(x)
    y = np.empty_like(x)
    yn = np.empty_like(x) if want_norm else None
    st = np.empty((B * T, STATS_PER_ROW), np.float32) if want_stats else None
    rc = lib.oracle_residual_gate_rmsnorm_scale_shift(
        _ptr(res), _ptr(x), _ptr(g), _ptr(weight), _ptr(sc), _ptr(sh), _ptr(r), _ptr(y), B, T, H,
        gbs, sbs, hbs, float(np.float32(eps)), _ptr(yn), _ptr(st))
    _check(rc, "residual_gate_rmsnorm_scale_shift")
    out = (r,) + _ret(y, yn, st, want_norm, want_stats, tup=True)
    return out


def residual_gate_layernorm_modulate(res, x, gate, scale, shift, eps=1e-6, want_norm=False,
                                     want_stats=False):
    """r = res + gate[b]*x (two roundings); y = LN(r)*(1+scale[b])+shift[b].
    Returns (r, y[, yn][, stats]); stats are the LN statistics of r."""
    lib = _load()
    res = _act(res, "res")
    x = _act(x, "x")
    if res.shape != x.shape:
        raise ValueError("res and x shapes differ")
    B, T, H = x.shape
    g, gbs = _vec(gate, B, H, "gate")
    sc, sbs = _vec(scale, B, H, "scale")
    sh, hbs = _vec(shift, B, H, "shift")
    r = np.empty_like(x)
    y = np.empty_like(x)
    yn = np.empty_like(x) if want_norm else None
    st = np.empty((B * T, STATS_PER_ROW), np.float32) if want_stats else None
    rc = lib.oracle_residual_gate_layernorm_modulate(
        _ptr(res), _ptr(x), _ptr(g), _ptr(sc), _ptr(sh), _ptr(r), _ptr(y), B, T, H, gbs, sbs, hbs,
        float(np.float32(eps)), _ptr(yn), _ptr(st))
    _check(rc, "residual_gate_layernorm_modulate")
    return (r,) + _ret(y, yn, st, want_norm, want_stats, tup=True)


def layernorm_modulate_fp8(x, scale, shift, qscale, eps=1e-6, want_y=False, want_stats=False):
    """q = e4m3fn(clamp(RN(f(y) * RN(1/qscale)), -448, 448)) of the LayerNorm+modulate
    output y; uint8 codes [B,T,H].  Returns q[, y][, stats]."""
    lib = _load()
    x = _act(x, "x")
    B, T, H = x.shape
    sc, sbs = _vec(scale, B, H, "scale")
    sh, hbs = _vec(shift, B, H, "shift")
    q = np.empty(x.shape, np.uint8)
    y = np.empty_like(x) if want_y else None
    st = np.empty((B * T, STATS_PER_ROW), np.float32) if want_stats else None
    rc = lib.oracle_layernorm_modulate_fp8(_ptr(x), _ptr(sc), _ptr(sh), float(np.float32(qscale)),
                                           _ptr(q), B, T, H, sbs, hbs, float(np.float32(eps)),
                                           _ptr(y), _ptr(st))
    _check(rc, "layernorm_modulate_fp8")
    return _ret(q, y, st, want_y, want_stats)


def to_e4m3fn(a):
    """Elementwise binary32 -> OCP E4M3 (e4m3fn) codes, nearest-even, no clamping."""
    lib = _load()
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint8)
    lib.oracle_to_e4m3fn(_ptr(a), _ptr(out), a.size)
    return out


def quant_fp8(y, qscale):
    """Elementwise static quantisation of bf16 bits y with scale qscale."""
    lib = _load()
    y = np.ascontiguousarray(y, dtype=np.uint16)
    out = np.empty(y.shape, np.uint8)
    lib.oracle_quant_fp8(_ptr(y), _ptr(out), y.size, float(np.float32(qscale)))
    return out


def _heads(a, name, tokens=None):
    """A [tokens, heads, head_dim] uint16 view with unit head_dim stride and head stride
    head_dim (token stride free); returns (array, heads, token stride in elements)."""
    a = np.asarray(a)
    if a.dtype != np.uint16 or a.ndim != 3 or a.strides[2] != 2 or a.strides[1] != 2 * a.shape[2]:
        raise ValueError(f"{name}: expected [tokens, heads, head_dim] with contiguous heads")
    if tokens is not None and a.shape[0] != tokens:
        raise ValueError(f"{name}: token count differs")
    return a, a.shape[1], a.strides[0] // 2


def qk_rmsnorm_rope(q, k, q_weight, k_weight, cos_sin, eps=1e-6, want_norm=False):
    """Per-head RMSNorm of q and k, then interleaved RoPE; returns (q_out, k_out[, yn_q,
    yn_k]).  q, k: [tokens, heads, head_dim] (token stride free, e.g. views of a packed
    QKV row); cos_sin: float32 [tokens, head_dim] (cos half, then sin half)."""
    lib = _load()
    q, hq, qts = _heads(q, "q")
    T, _, D = q.shape
    k, hk, kts = _heads(k, "k", T)
    if k.shape[2] != D:
        raise ValueError("q and k head_dim differ")
    cs = np.ascontiguousarray(cos_sin, dtype=np.float32).reshape(T, D)
    qw = None if q_weight is None else np.ascontiguousarray(q_weight, np.uint16).reshape(D)
    kw = None if k_weight is None else np.ascontiguousarray(k_weight, np.uint16).reshape(D)
    qo = np.empty((T, hq, D), np.uint16)
    ko = np.empty((T, hk, D), np.uint16)
    ynq = np.empty_like(qo) if want_norm else None
    ynk = np.empty_like(ko) if want_norm else None
    base_q = q.ctypes.data
    base_k = k.ctypes.data
    rc = lib.oracle_qk_rmsnorm_rope(base_q, base_k, _ptr(qw), _ptr(kw), _ptr(cs), _ptr(qo),
                                    _ptr(ko), T, hq, hk, D, qts, kts, float(np.float32(eps)),
                                    _ptr(ynq), _ptr(ynk))
    _check(rc, "qk_rmsnorm_rope")
    return (qo, ko, ynq, ynk) if want_norm else (qo, ko)


def residual_gate_channel_first(res, update, gate):
    """out[b,h,t] = round(res[b,h,t] + round(gate[b,h] * update[b,t,h])); res and out
    [B,H,T] (channel-first), update [B,T,H]."""
    lib = _load()
    res = np.ascontiguousarray(res, np.uint16)
    update = np.ascontiguousarray(update, np.uint16)
    B, H, T = res.shape
    if update.shape != (B, T, H):
        raise ValueError("update must be [B, T, H] for res [B, H, T]")
    g, gbs = _vec(gate, B, H, "gate")
    out = np.empty_like(res)
    rc = lib.oracle_residual_gate_channel_first(_ptr(res), _ptr(update), _ptr(g), _ptr(out), B, T,
                                                H, gbs)
    _check(rc, "residual_gate_channel_first")
    return out


def _ret(y, yn, st, want_norm, want_stats, tup=False):
    out = (y,)
    if want_norm:
        out += (yn,)
    if want_stats:
        out += (st,)
    if tup:
        return out
    return out[0] if len(out) == 1 else out


def round_bf16(a):
    """Elementwise binary32 -> bf16 bits, nearest-even."""
    lib = _load()
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint16)
    lib.oracle_round_bf16(_ptr(a), _ptr(out), a.size)
    return out


def modulate(yn, scale, shift):
    """Elementwise round(round(yn * round(1 + scale)) + shift) on bf16 bits."""
    lib = _load()
    yn, scale, shift = (np.ascontiguousarray(v, dtype=np.uint16) for v in (yn, scale, shift))
    out = np.empty(yn.shape, np.uint16)
    lib.oracle_modulate(_ptr(yn), _ptr(scale), _ptr(shift), _ptr(out), yn.size)
    return out


def gate_residual(res, x, gate):
    """Elementwise round(res + round(gate * x)) on bf16 bits."""
    lib = _load()
    res, x, gate = (np.ascontiguousarray(v, dtype=np.uint16) for v in (res, x, gate))
    out = np.empty(res.shape, np.uint16)
    lib.oracle_gate_residual(_ptr(res), _ptr(x), _ptr(gate), _ptr(out), res.size)
    return out
