"""ctypes binding of libadaln (include/adaln.h): argument marshalling only.

Torch tensors supply device pointers, strides and the current HIP stream; every
step of the computation runs in the library's HIP kernels.  A missing library is
an error (no CPU fallback exists).
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
ABI_VERSION = 11

STATUS_NAMES = {0: "ADALN_OK", 1: "ADALN_ERR_NULL", 2: "ADALN_ERR_SHAPE", 3: "ADALN_ERR_ALIGN",
                4: "ADALN_ERR_STRIDE", 5: "ADALN_ERR_OVERLAP", 6: "ADALN_ERR_VALUE",
                7: "ADALN_ERR_LAUNCH"}

# every symbol include/adaln.h declares
EXPORTS = ("adaln_layernorm_modulate", "adaln_rmsnorm_scale_shift",
           "adaln_residual_gate_rmsnorm_scale_shift", "adaln_residual_gate_layernorm_modulate",
           "adaln_layernorm_modulate_fp8_quant", "adaln_qk_rmsnorm_rope",
           "adaln_residual_gate_channel_first", "adaln_check_layernorm_modulate",
           "adaln_check_qk_rmsnorm_rope", "adaln_check_residual_gate_channel_first",
           "adaln_check_rmsnorm_scale_shift", "adaln_check_residual_gate_rmsnorm_scale_shift",
           "adaln_check_residual_gate_layernorm_modulate",
           "adaln_check_layernorm_modulate_fp8_quant", "adaln_reduction_layout",
           "adaln_status_string", "adaln_abi_version", "adaln_diag_round_bf16",
           "adaln_diag_finalize", "adaln_diag_quant_fp8", "adaln_diag_stream_copy",
           "adaln_diag_stream", "adaln_diag_launch_plan", "adaln_diag_device_plan")


class AdalnError(RuntimeError):
    """A libadaln entry point returned a non-OK status."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({_status_text(status)})")


_lib = None


def library_path() -> str:
    """The in-tree libadaln.so (the only library the binding loads)."""
    return os.path.join(_PKG, "libadaln.so")


def load_library():
    """Load the built libadaln.so from the package directory (raises if absent)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libadaln is not built ({path} missing); run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    sig = {
        "adaln_layernorm_modulate": [P, P, P, P, I, I, I, I, I, F, P],
        "adaln_rmsnorm_scale_shift": [P, P, P, P, P, I, I, I, I, I, F, P],
        "adaln_residual_gate_rmsnorm_scale_shift": [P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, P],
        "adaln_residual_gate_layernorm_modulate": [P, P, P, P, P, P, P, I, I, I, I, I, I, F, P],
        "adaln_layernorm_modulate_fp8_quant": [P, P, P, P, P, I, I, I, I, I, F, P],
        "adaln_check_layernorm_modulate_fp8_quant": [P, P, P, P, P, I, I, I, I, I, F],
        "adaln_qk_rmsnorm_rope": [P, P, P, P, P, P, P, I, I, I, I, I, I, F, P],
        "adaln_check_qk_rmsnorm_rope": [P, P, P, P, P, P, P, I, I, I, I, I, I, F],
        "adaln_residual_gate_channel_first": [P, P, P, P, I, I, I, I, P],
        "adaln_check_residual_gate_channel_first": [P, P, P, P, I, I, I, I],
        "adaln_check_layernorm_modulate": [P, P, P, P, I, I, I, I, I, F],
        "adaln_check_rmsnorm_scale_shift": [P, P, P, P, P, I, I, I, I, I, F],
        "adaln_check_residual_gate_rmsnorm_scale_shift": [P, P, P, P, P, P, P, P, I, I, I, I, I, I,
                                                          F],
        "adaln_check_residual_gate_layernorm_modulate": [P, P, P, P, P, P, P, I, I, I, I, I, I, F],
        "adaln_reduction_layout": [I, ctypes.POINTER(S), ctypes.POINTER(S), ctypes.POINTER(S)],
        "adaln_diag_round_bf16": [P, P, I, P],
        "adaln_diag_finalize": [P, P, I, I, F, P],
        "adaln_diag_stream_copy": [P, P, I, P],
        "adaln_diag_stream": [S, P, P, I, S, P],
        "adaln_diag_quant_fp8": [P, P, I, P, P],
        "adaln_diag_launch_plan": [S, I, I, I, ctypes.POINTER(I), I, ctypes.POINTER(I)],
        "adaln_diag_device_plan": [S, I, I, I, S, ctypes.POINTER(I), ctypes.POINTER(I),
                                   ctypes.POINTER(I)],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = S
    lib.adaln_status_string.argtypes = [S]
    lib.adaln_status_string.restype = ctypes.c_char_p
    lib.adaln_abi_version.argtypes = []
    lib.adaln_abi_version.restype = S
    if lib.adaln_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libadaln ABI {lib.adaln_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = lib
    return lib


def _status_text(status: int) -> str:
    try:
        return load_library().adaln_status_string(int(status)).decode()
    except Exception:  # pragma: no cover - library missing while formatting an error
        return "?"


def _check(status: int, what: str):
    if status != 0:
        raise AdalnError(status, what)


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _act(t: torch.Tensor, name: str, shape=None):
    if t.dtype != torch.bfloat16 or t.dim() != 3 or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous bfloat16 [B,T,H] tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _on(dev, *named):
    """Every given tensor must live on the GPU `dev` (the library takes device
    pointers only; a host pointer or another GPU's memory would be dereferenced by
    the kernel)."""
    if dev.type != "cuda":
        raise ValueError(f"expected CUDA (HIP) tensors, got a tensor on {dev}")
    for t, name in named:
        if t is not None and (not isinstance(t, torch.Tensor) or t.device != dev):
            raise ValueError(f"{name}: expected a tensor on {dev}")


def _call(dev, fn, *args, stream=None):
    """Call a library entry point with `dev` current (its stream argument last)."""
    with torch.cuda.device(dev):
        return fn(*args, _stream(stream))


def _vec(v: torch.Tensor, B: int, H: int, name: str):
    """Pointer and batch stride (elements) of a per-batch vector [B,H], [1,H] or [H]."""
    if v.dtype != torch.bfloat16:
        raise ValueError(f"{name}: expected bfloat16")
    if v.dim() == 1:
        v = v.unsqueeze(0)
    if v.dim() != 2 or v.size(1) != H or v.stride(1) != 1 or v.size(0) not in (1, B):
        raise ValueError(f"{name}: expected [B,H], [1,H] or [H] with unit inner stride")
    bstride = v.stride(0) if (v.size(0) == B and B > 1) else 0
    return v.data_ptr(), bstride


def _ptr(t):
    return None if t is None else t.data_ptr()


def _eps(eps: float) -> float:
    return float(torch.tensor(eps, dtype=torch.float32).item())


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def adaln_layernorm_modulate(x, scale, shift, eps: float = 1e-6, out=None, stream=None):
    """y = LayerNorm(x) * (1 + scale[b]) + shift[b] (no affine)."""
    lib = load_library()
    _act(x, "x")
    B, T, H = x.shape
    _on(x.device, (scale, "scale"), (shift, "shift"), (out, "out"))
    sp, sbs = _vec(scale, B, H, "scale")
    hp, hbs = _vec(shift, B, H, "shift")
    y = torch.empty_like(x) if out is None else _act(out, "out", x.shape)
    _check(_call(x.device, lib.adaln_layernorm_modulate, x.data_ptr(), sp, hp, y.data_ptr(), B, T,
                 H, sbs, hbs, _eps(eps), stream=stream), "adaln_layernorm_modulate")
    return y


def adaln_rmsnorm_scale_shift(x, weight, scale, shift, eps: float = 1e-6, out=None, stream=None):
    """y = RMSNorm(x) * (1 + scale[b]) + shift[b]; weight None means one."""
    lib = load_library()
    _act(x, "x")
    B, T, H = x.shape
    if weight is not None and (weight.dtype != torch.bfloat16 or weight.numel() != H
                               or not weight.is_contiguous()):
        raise ValueError("weight: expected a contiguous bfloat16 [H] tensor")
    _on(x.device, (weight, "weight"), (scale, "scale"), (shift, "shift"), (out, "out"))
    sp, sbs = _vec(scale, B, H, "scale")
    hp, hbs = _vec(shift, B, H, "shift")
    y = torch.empty_like(x) if out is None else _act(out, "out", x.shape)
    _check(_call(x.device, lib.adaln_rmsnorm_scale_shift, x.data_ptr(), _ptr(weight), sp, hp,
                 y.data_ptr(), B, T, H, sbs, hbs, _eps(eps), stream=stream),
           "adaln_rmsnorm_scale_shift")
    return y


def adaln_residual_gate_rmsnorm_scale_shift(res, x, gate, weight, scale, shift, eps: float = 1e-6,
                                            out=None, r_out=None, stream=None):
    """(r, y): r = res + gate[b] * x, y = RMSNorm(r) * (1 + scale[b]) + shift[b]."""
    lib = load_library()
    _act(res, "res")
    _act(x, "x")
    if res.shape != x.shape:
        raise ValueError("res and x must have the same shape")
    B, T, H = x.shape
    if weight is not None and (weight.dtype != torch.bfloat16 or weight.numel() != H
                               or not weight.is_contiguous()):
        raise ValueError("weight: expected a contiguous bfloat16 [H] tensor")
    _on(x.device, (res, "res"), (gate, "gate"), (weight, "weight"), (scale, "scale"),
        (shift, "shift"), (out, "out"), (r_out, "r_out"))
    gp, gbs = _vec(gate, B, H, "gate")
    sp, sbs = _vec(scale, B, H, "scale")
    hp, hbs = _vec(shift, B, H, "shift")
    y = torch.empty_like(x) if out is None else _act(out, "out", x.shape)
    r = torch.empty_like(x) if r_out is None else _act(r_out, "r_out", x.shape)
    _check(_call(x.device, lib.adaln_residual_gate_rmsnorm_scale_shift, res.data_ptr(),
                 x.data_ptr(), gp, _ptr(weight), sp, hp, r.data_ptr(), y.data_ptr(), B, T, H, gbs,
                 sbs, hbs, _eps(eps), stream=stream), "adaln_residual_gate_rmsnorm_scale_shift")
    return r, y


def adaln_residual_gate_layernorm_modulate(res, x, gate, scale, shift, eps: float = 1e-6,
                                           out=None, r_out=None, stream=None):
    """(r, y): r = res + gate[b] * x, y = LayerNorm(r) * (1 + scale[b]) + shift[b]."""
    lib = load_library()
    _act(res, "res")
    _act(x, "x")
    if res.shape != x.shape:
        raise ValueError("res and x must have the same shape")
    B, T, H = x.shape
    _on(x.device, (res, "res"), (gate, "gate"), (scale, "scale"), (shift, "shift"),
        (out, "out"), (r_out, "r_out"))
    gp, gbs = _vec(gate, B, H, "gate")
    sp, sbs = _vec(scale, B, H, "scale")
    hp, hbs = _vec(shift, B, H, "shift")
    y = torch.empty_like(x) if out is None else _act(out, "out", x.shape)
    r = torch.empty_like(x) if r_out is None else _act(r_out, "r_out", x.shape)
    _check(_call(x.device, lib.adaln_residual_gate_layernorm_modulate, res.data_ptr(),
                 x.data_ptr(), gp, sp, hp, r.data_ptr(), y.data_ptr(), B, T, H, gbs, sbs, hbs,
                 _eps(eps), stream=stream), "adaln_residual_gate_layernorm_modulate")
    return r, y


def adaln_layernorm_modulate_fp8_quant(x, scale, shift, qscale, eps: float = 1e-6, out=None,
                                       stream=None):
    """q (uint8 E4M3 codes [B,T,H]) = static FP8 quantisation of
    LayerNorm(x) * (1 + scale[b]) + shift[b]; qscale is a one-element float32 device
    tensor (the per-tensor input scale).  View q as torch.float8_e4m3fn if wanted."""
    lib = load_library()
    _act(x, "x")
    B, T, H = x.shape
    _on(x.device, (scale, "scale"), (shift, "shift"), (qscale, "qscale"), (out, "out"))
    if qscale.dtype != torch.float32 or qscale.numel() != 1:
        raise ValueError("qscale: expected a one-element float32 device tensor")
    sp, sbs = _vec(scale, B, H, "scale")
    hp, hbs = _vec(shift, B, H, "shift")
    if out is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    else:
        if out.dtype != torch.uint8 or out.shape != x.shape or not out.is_contiguous():
            raise ValueError("out: expected a contiguous uint8 [B,T,H] tensor")
        q = out
    _check(_call(x.device, lib.adaln_layernorm_modulate_fp8_quant, x.data_ptr(), sp, hp,
                 qscale.data_ptr(), q.data_ptr(), B, T, H, sbs, hbs, _eps(eps), stream=stream),
           "adaln_layernorm_modulate_fp8_quant")
    return q


def _heads_view(t: torch.Tensor, name: str):
    if (t.dtype != torch.bfloat16 or t.dim() != 3 or t.size(2) != 128 or t.stride(2) != 1
            or t.stride(1) != 128):
        raise ValueError(f"{name}: expected bfloat16 [tokens, heads, 128] with contiguous heads")
    return t.stride(0)


def adaln_qk_rmsnorm_rope(q, k, q_weight, k_weight, cos_sin, eps: float = 1e-6, q_out=None,
                          k_out=None, stream=None):
    """(q_out, k_out): per-head RMSNorm of q and k ([tokens, heads, 128], e.g. views
    of a packed QKV row) with their weights, then interleaved RoPE from cos_sin
    (float32 [tokens, 128]: cos of the 64 pairs, then sin)."""
    lib = load_library()
    qts = _heads_view(q, "q")
    kts = _heads_view(k, "k")
    T = q.size(0)
    if k.size(0) != T:
        raise ValueError("q and k token counts differ")
    if cos_sin.dtype != torch.float32 or cos_sin.shape != (T, 128) or not cos_sin.is_contiguous():
        raise ValueError("cos_sin: expected a contiguous float32 [tokens, 128] tensor")
    for w, name in ((q_weight, "q_weight"), (k_weight, "k_weight")):
        if w is not None and (w.dtype != torch.bfloat16 or w.numel() != 128 or
                              not w.is_contiguous()):
            raise ValueError(f"{name}: expected a contiguous bfloat16 [128] tensor")
    _on(q.device, (k, "k"), (q_weight, "q_weight"), (k_weight, "k_weight"),
        (cos_sin, "cos_sin"), (q_out, "q_out"), (k_out, "k_out"))
    qo = torch.empty((T, q.size(1), 128), dtype=torch.bfloat16, device=q.device) \
        if q_out is None else _act(q_out, "q_out", (T, q.size(1), 128))
    ko = torch.empty((T, k.size(1), 128), dtype=torch.bfloat16, device=k.device) \
        if k_out is None else _act(k_out, "k_out", (T, k.size(1), 128))
    _check(_call(q.device, lib.adaln_qk_rmsnorm_rope, q.data_ptr(), k.data_ptr(), _ptr(q_weight),
                 _ptr(k_weight), cos_sin.data_ptr(), qo.data_ptr(), ko.data_ptr(), T, q.size(1),
                 k.size(1), 128, qts, kts, _eps(eps), stream=stream), "adaln_qk_rmsnorm_rope")
    return qo, ko


def adaln_residual_gate_channel_first(res, update, gate, out=None, stream=None):
    """out[b,h,t] = res[b,h,t] + gate[b,h] * update[b,t,h] (two bf16 roundings); res and
    out contiguous [B,H,T] (channel-first), update contiguous [B,T,H].  out=res updates
    the residual in place."""
    lib = load_library()
    if res.dtype != torch.bfloat16 or res.dim() != 3 or not res.is_contiguous():
        raise ValueError("res: expected a contiguous bfloat16 [B,H,T] tensor")
    B, H, T = res.shape
    if (update.dtype != torch.bfloat16 or tuple(update.shape) != (B, T, H)
            or not update.is_contiguous()):
        raise ValueError("update: expected a contiguous bfloat16 [B,T,H] tensor")
    _on(res.device, (update, "update"), (gate, "gate"), (out, "out"))
    gp, gbs = _vec(gate, B, H, "gate")
    o = torch.empty_like(res) if out is None else out
    if o.shape != res.shape or o.dtype != torch.bfloat16 or not o.is_contiguous():
        raise ValueError("out: expected a contiguous bfloat16 [B,H,T] tensor")
    _check(_call(res.device, lib.adaln_residual_gate_channel_first, res.data_ptr(),
                 update.data_ptr(), gp, o.data_ptr(), B, T, H, gbs, stream=stream),
           "adaln_residual_gate_channel_first")
    return o


def adaln_check_layernorm_modulate(x_ptr, scale_ptr, shift_ptr, y_ptr, B, T, H, scale_bstride,
                                   shift_bstride, eps=1e-6) -> int:
    """Status code of the validation (raw pointers as ints; nothing is launched)."""
    return load_library().adaln_check_layernorm_modulate(x_ptr, scale_ptr, shift_ptr, y_ptr, B, T,
                                                         H, scale_bstride, shift_bstride, eps)


def adaln_check_rmsnorm_scale_shift(x_ptr, weight_ptr, scale_ptr, shift_ptr, y_ptr, B, T, H,
                                    scale_bstride, shift_bstride, eps=1e-6) -> int:
    return load_library().adaln_check_rmsnorm_scale_shift(x_ptr, weight_ptr, scale_ptr, shift_ptr,
                                                          y_ptr, B, T, H, scale_bstride,
                                                          shift_bstride, eps)


def adaln_check_residual_gate_rmsnorm_scale_shift(res_ptr, x_ptr, gate_ptr, weight_ptr, scale_ptr,
                                                  shift_ptr, r_ptr, y_ptr, B, T, H, gate_bstride,
                                                  scale_bstride, shift_bstride, eps=1e-6) -> int:
    return load_library().adaln_check_residual_gate_rmsnorm_scale_shift(
        res_ptr, x_ptr, gate_ptr, weight_ptr, scale_ptr, shift_ptr, r_ptr, y_ptr, B, T, H,
        gate_bstride, scale_bstride, shift_bstride, eps)


def adaln_check_residual_gate_layernorm_modulate(res_ptr, x_ptr, gate_ptr, scale_ptr, shift_ptr,
                                                 r_ptr, y_ptr, B, T, H, gate_bstride,
                                                 scale_bstride, shift_bstride, eps=1e-6) -> int:
    return load_library().adaln_check_residual_gate_layernorm_modulate(
        res_ptr, x_ptr, gate_ptr, scale_ptr, shift_ptr, r_ptr, y_ptr, B, T, H, gate_bstride,
        scale_bstride, shift_bstride, eps)


def adaln_check_layernorm_modulate_fp8_quant(x_ptr, scale_ptr, shift_ptr, qscale_ptr, q_ptr, B, T,
                                             H, scale_bstride, shift_bstride, eps=1e-6) -> int:
    return load_library().adaln_check_layernorm_modulate_fp8_quant(
        x_ptr, scale_ptr, shift_ptr, qscale_ptr, q_ptr, B, T, H, scale_bstride, shift_bstride, eps)


def adaln_check_qk_rmsnorm_rope(q_ptr, k_ptr, q_weight_ptr, k_weight_ptr, cos_sin_ptr, q_out_ptr,
                                k_out_ptr, tokens, heads_q, heads_k, head_dim, q_token_stride,
                                k_token_stride, eps=1e-6) -> int:
    return load_library().adaln_check_qk_rmsnorm_rope(
        q_ptr, k_ptr, q_weight_ptr, k_weight_ptr, cos_sin_ptr, q_out_ptr, k_out_ptr, tokens,
        heads_q, heads_k, head_dim, q_token_stride, k_token_stride, eps)


def adaln_check_residual_gate_channel_first(res_ptr, update_ptr, gate_ptr, out_ptr, B, T, H,
                                            gate_bstride) -> int:
    return load_library().adaln_check_residual_gate_channel_first(res_ptr, update_ptr, gate_ptr,
                                                                  out_ptr, B, T, H, gate_bstride)


def adaln_reduction_layout(H: int):
    """(waves per row, lanes per row, chunks per lane) of the fixed order for H."""
    lib = load_library()
    w, p, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib.adaln_reduction_layout(H, ctypes.byref(w), ctypes.byref(p), ctypes.byref(c)),
           "adaln_reduction_layout")
    return w.value, p.value, c.value


OPS = {"ln": 0, "rms": 1, "rg": 2, "rgln": 3, "lnq": 4}
PLAN_FIELDS = ("shallow", "slots", "ring", "groups", "gpb", "blk_rows", "group_stride", "step",
               "span", "blocks", "block_threads")


def adaln_diag_launch_plan(op: str, rows: int, H: int, T: int, resident, cus: int = 0) -> dict:
    """The fused launch's row-group plan for B = rows / T batch entries, given what fits
    on the device at once (host only; see the header): resident = (groups with the
    default ring, with the one-slot ring, with the two-row ring); missing trailing
    counts are 0, so a single number n means (n, 0, 0)."""
    lib = load_library()
    if isinstance(resident, int):
        resident = (resident,)
    if len(resident) > 3:
        raise ValueError("at most three resident counts")
    res = (ctypes.c_int64 * 3)(*(list(resident) + [0] * (3 - len(resident))))
    out = (ctypes.c_int64 * len(PLAN_FIELDS))()
    _check(lib.adaln_diag_launch_plan(OPS[op], rows, H, T, res, cus, out),
           "adaln_diag_launch_plan")
    return dict(zip(PLAN_FIELDS, list(out)))


def adaln_diag_device_plan(op: str, rows: int, H: int, T: int, weight: bool = False) -> dict:
    """The plan a launch on the current device takes, with the resident counts and CU
    count it was made from (keys "resident", "cus")."""
    lib = load_library()
    out = (ctypes.c_int64 * len(PLAN_FIELDS))()
    res = (ctypes.c_int64 * 3)()
    cus = ctypes.c_int64()
    _check(lib.adaln_diag_device_plan(OPS[op], rows, H, T, int(bool(weight)), out, res,
                                      ctypes.byref(cus)), "adaln_diag_device_plan")
    d = dict(zip(PLAN_FIELDS, list(out)))
    d["resident"] = tuple(res)
    d["cus"] = cus.value
    return d


def adaln_status_string(status: int) -> str:
    return load_library().adaln_status_string(int(status)).decode()


def adaln_abi_version() -> int:
    return load_library().adaln_abi_version()


def adaln_diag_round_bf16(x: torch.Tensor, stream=None) -> torch.Tensor:
    """Device bf16 rounding of a float32 tensor (the kernels' rounding step)."""
    lib = load_library()
    if x.dtype != torch.float32 or not x.is_contiguous():
        raise ValueError("expected a contiguous float32 tensor")
    _on(x.device)
    out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    _check(_call(x.device, lib.adaln_diag_round_bf16, x.data_ptr(), out.data_ptr(), x.numel(),
                 stream=stream), "adaln_diag_round_bf16")
    return out


def adaln_diag_finalize(x: torch.Tensor, eps: float = 1e-6, H: int = 1,
                        stream=None) -> torch.Tensor:
    """Device rstd = RN(1/RN(sqrt(RN(RN(x / H) + eps)))) of a float32 tensor of row
    statistics over H elements (the kernels' step)."""
    lib = load_library()
    if x.dtype != torch.float32 or not x.is_contiguous():
        raise ValueError("expected a contiguous float32 tensor")
    _on(x.device)
    out = torch.empty_like(x)
    _check(_call(x.device, lib.adaln_diag_finalize, x.data_ptr(), out.data_ptr(), x.numel(),
                 int(H), _eps(eps), stream=stream), "adaln_diag_finalize")
    return out


def adaln_diag_stream_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> torch.Tensor:
    """Copy src into dst (same byte size, contiguous) with the library's streaming copy."""
    lib = load_library()
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("expected contiguous tensors")
    _on(src.device, (dst, "dst"))
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst sizes differ")
    _check(_call(src.device, lib.adaln_diag_stream_copy, src.data_ptr(), dst.data_ptr(), nbytes,
                 stream=stream), "adaln_diag_stream_copy")
    return dst


STREAM_KINDS = {"copy": 0, "read": 1, "fill": 2}


def adaln_diag_stream(kind: str, src, dst: torch.Tensor, vectors_per_thread: int = 8,
                      stream=None) -> None:
    """The library's streaming measurement kernel `kind` (copy, read or fill) over the
    byte size of dst (contiguous; src the same size, or None for fill)."""
    lib = load_library()
    if not dst.is_contiguous() or (src is not None and not src.is_contiguous()):
        raise ValueError("expected contiguous tensors")
    _on(dst.device, (src, "src"))
    nbytes = dst.numel() * dst.element_size()
    if src is not None and src.numel() * src.element_size() != nbytes:
        raise ValueError("src and dst sizes differ")
    _check(_call(dst.device, lib.adaln_diag_stream, STREAM_KINDS[kind], _ptr(src),
                 dst.data_ptr(), nbytes, int(vectors_per_thread), stream=stream),
           "adaln_diag_stream")


def adaln_diag_quant_fp8(v: torch.Tensor, qscale: torch.Tensor, stream=None) -> torch.Tensor:
    """The FP8 kernel's quantisation step on a float32 tensor (numel % 4 == 0)."""
    lib = load_library()
    if v.dtype != torch.float32 or not v.is_contiguous():
        raise ValueError("expected a contiguous float32 tensor")
    _on(v.device, (qscale, "qscale"))
    if qscale.dtype != torch.float32 or qscale.numel() != 1:
        raise ValueError("qscale: expected a one-element float32 device tensor")
    out = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    _check(_call(v.device, lib.adaln_diag_quant_fp8, v.data_ptr(), out.data_ptr(), v.numel(),
                 qscale.data_ptr(), stream=stream), "adaln_diag_quant_fp8")
    return out
