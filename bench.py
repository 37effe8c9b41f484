"""Benchmark of the fused adaLN path on one MI355X.

A step is one pass of the whole hot path (load, statistic, fold, finalize,
normalise, modulate, store) over one batch: one launch of the fused kernel.  The
metric names no single configuration, so the timed line is the largest of them that
has a bandwidth target: LayerNorm + modulate on bf16 x [2, 4608, 3072] (the FLUX.1
adaLN site with CFG batch 2).  Inputs are resident in HBM; the launches rotate over
buffer sets totalling >= 1 GiB so every launch reads from HBM, not from the 256 MB
Infinity Cache.

Prints ONE JSON line: value = achieved HBM GB/s (algorithmic bytes: read x[,res],
write y[,r]) over the timed steps, plus rows/s and the roofline of the fused
kernel; then, per configuration with the 80 %-of-peak target (RMSNorm [1,4216,4096],
residual-gate RMSNorm [2,1140,4096], LayerNorm [2,4608,3072] and [1,4333,3072]), its
own roofline object: events and kernel-trace time, fraction of the 8 TB/s peak,
HBM traffic ratio, and fractions of the measured streaming ceilings (copy, read-only,
write-only at the same bytes and at 1 GiB); the other workloads' figures; and the
CPU oracle timed on this host as the baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "achieved HBM GB/s (% of MI355X peak) and rows/s for fused norm+modulate"
# the sources of the kernels whose profiles are committed (the fused template, the
# QK and channel-first kernels, the streaming kernels, shared helpers, parameters)
KERNEL_SRCS = [os.path.join(ROOT, "diffusion_dit_adaln_amd", "csrc", f)
               for f in ("adaln_kernels.hip", "adaln_qknorm.hip", "adaln_channel_first.hip",
                         "adaln_stream.hip", "adaln_device.hpp", "adaln_fold.hpp",
                         "adaln_internal.hpp")]


def kernel_src_sha() -> str:
    """Hash of the fused kernel's code: its sources with comments and blank space
    removed, so that a comment edit does not invalidate the counters."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_counters(name: str):
    """Per-dispatch HBM bytes from the committed rocprofv3 --pmc summary, or None
    when the summary is missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"counters_{name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_src_sha") != kernel_src_sha():
        return None
    try:
        return float(kv["traffic_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
HEADLINE = "ln_2x4608x3072"
# the configurations of the metric that carry the 80 %-of-peak target
TARGET_CONFIGS = ["rms_1x4216x4096", "rg_rms_2x1140x4096", "ln_2x4608x3072", "ln_1x4333x3072"]
TARGET_FRAC = 0.80
STREAM_PERS = (1, 2, 4, 8, 16)
WORKLOAD_NAMES = ["ln_1x128x2048", "rms_1x4216x4096", "rg_rms_2x1140x4096", "ln_2x4608x3072",
                  "ln_1x4333x3072", "rg_ln_2x4096x3072", "ln_fp8_2x4608x3072",
                  "qk_rmsnorm_rope_4608x24x128", "rg_channel_first_2x3072x4608"]


def workload(name: str):
    from diffusion_dit_adaln_amd import synth
    return synth.WORKLOADS[name]()


class Launcher:
    """Pre-marshalled C-ABI calls over rotating device buffer sets."""

    def __init__(self, wl, rotate_bytes: int):
        import torch
        import diffusion_dit_adaln_amd as A
        self.torch = torch
        self.lib = A.load_library()
        self.wl = wl
        B, T, H = wl.x.shape
        self.B, self.T, self.H = B, T, H

        def dev(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).cuda()

        per_set = wl.algorithmic_bytes()
        self.nsets = max(2, -(-rotate_bytes // per_set))
        x0 = dev(wl.x)
        self.sets = []
        for _ in range(self.nsets):
            if wl.op == "lnq":
                s = {"x": x0.clone(), "y": torch.empty(x0.shape, dtype=torch.uint8, device="cuda")}
            else:
                s = {"x": x0.clone(), "y": torch.empty_like(x0)}
            if wl.op in ("rg", "rgln"):
                s["res"] = dev(wl.res)
                s["r"] = torch.empty_like(x0)
            self.sets.append(s)
        self.scale = dev(wl.scale)
        self.shift = dev(wl.shift)
        self.weight = dev(wl.weight) if wl.weight is not None else None
        self.gate = dev(wl.gate) if wl.gate is not None else None
        self.qscale = (torch.tensor([wl.qscale], dtype=torch.float32, device="cuda")
                       if wl.qscale is not None else None)
        self.eps = ctypes.c_float(np.float32(wl.eps))
        bs = H if B > 1 else 0
        self.bs = bs
        del x0
        torch.cuda.synchronize()

    def call(self, i: int, stream) -> int:
        s = self.sets[i % self.nsets]
        B, T, H, bs = self.B, self.T, self.H, self.bs
        if self.wl.op == "ln":
            return self.lib.adaln_layernorm_modulate(
                s["x"].data_ptr(), self.scale.data_ptr(), self.shift.data_ptr(), s["y"].data_ptr(),
                B, T, H, bs, bs, self.eps, stream)
        if self.wl.op == "rms":
            return self.lib.adaln_rmsnorm_scale_shift(
                s["x"].data_ptr(), None if self.weight is None else self.weight.data_ptr(),
                self.scale.data_ptr(), self.shift.data_ptr(), s["y"].data_ptr(), B, T, H, bs, bs,
                self.eps, stream)
        if self.wl.op == "lnq":
            return self.lib.adaln_layernorm_modulate_fp8_quant(
                s["x"].data_ptr(), self.scale.data_ptr(), self.shift.data_ptr(),
                self.qscale.data_ptr(), s["y"].data_ptr(), B, T, H, bs, bs, self.eps, stream)
        if self.wl.op == "rgln":
            return self.lib.adaln_residual_gate_layernorm_modulate(
                s["res"].data_ptr(), s["x"].data_ptr(), self.gate.data_ptr(),
                self.scale.data_ptr(), self.shift.data_ptr(), s["r"].data_ptr(),
                s["y"].data_ptr(), B, T, H, bs, bs, bs, self.eps, stream)
        return self.lib.adaln_residual_gate_rmsnorm_scale_shift(
            s["res"].data_ptr(), s["x"].data_ptr(), self.gate.data_ptr(),
            None if self.weight is None else self.weight.data_ptr(), self.scale.data_ptr(),
            self.shift.data_ptr(), s["r"].data_ptr(), s["y"].data_ptr(), B, T, H, bs, bs, bs,
            self.eps, stream)


class QKLauncher:
    """Pre-marshalled QK RMSNorm + RoPE calls over rotating packed-QKV buffer sets."""

    def __init__(self, wl, rotate_bytes: int):
        import torch
        import diffusion_dit_adaln_amd as A
        self.lib = A.load_library()
        self.wl = wl
        T, _, Hd, D = wl.qkv.shape
        self.T, self.Hd = T, Hd

        def dev(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).cuda()

        self.nsets = max(2, -(-rotate_bytes // wl.algorithmic_bytes()))
        q0 = dev(wl.qkv)
        self.sets = [{"qkv": q0.clone(), "qo": torch.empty((T, Hd, D), dtype=torch.bfloat16,
                                                            device="cuda"),
                      "ko": torch.empty((T, Hd, D), dtype=torch.bfloat16, device="cuda")}
                     for _ in range(self.nsets)]
        self.wq = dev(wl.q_weight)
        self.wk = dev(wl.k_weight)
        self.cs = torch.from_numpy(wl.cos_sin).cuda()
        self.eps = ctypes.c_float(np.float32(wl.eps))
        self.ts = 3 * Hd * D
        del q0
        torch.cuda.synchronize()

    def call(self, i: int, stream) -> int:
        s = self.sets[i % self.nsets]
        base = s["qkv"].data_ptr()
        row = self.Hd * 128 * 2
        return self.lib.adaln_qk_rmsnorm_rope(base, base + row, self.wq.data_ptr(),
                                              self.wk.data_ptr(), self.cs.data_ptr(),
                                              s["qo"].data_ptr(), s["ko"].data_ptr(), self.T,
                                              self.Hd, self.Hd, 128, self.ts, self.ts, self.eps,
                                              stream)


class CFLauncher:
    """Pre-marshalled channel-first residual-gate calls over rotating buffer sets."""

    def __init__(self, wl, rotate_bytes: int):
        import torch
        import diffusion_dit_adaln_amd as A
        self.lib = A.load_library()
        self.wl = wl
        self.B, self.H, self.T = wl.res.shape

        def dev(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).cuda()

        self.nsets = max(2, -(-rotate_bytes // wl.algorithmic_bytes()))
        r0, u0 = dev(wl.res), dev(wl.update)
        self.sets = [{"res": r0.clone(), "upd": u0.clone(), "out": torch.empty_like(r0)}
                     for _ in range(self.nsets)]
        self.gate = dev(wl.gate)
        del r0, u0
        torch.cuda.synchronize()

    def call(self, i: int, stream) -> int:
        s = self.sets[i % self.nsets]
        return self.lib.adaln_residual_gate_channel_first(
            s["res"].data_ptr(), s["upd"].data_ptr(), self.gate.data_ptr(), s["out"].data_ptr(),
            self.B, self.T, self.H, self.H if self.B > 1 else 0, stream)


def launcher_for(wl, rotate_bytes):
    if wl.op == "qk":
        return QKLauncher(wl, rotate_bytes)
    if wl.op == "cf":
        return CFLauncher(wl, rotate_bytes)
    return Launcher(wl, rotate_bytes)


def time_steps(launch, steps: int, warmup: int, mode: str):
    """Elapsed seconds of `steps` launches (warm-up excluded), timed with HIP
    events on the launch stream, bracketed by synchronize on both sides."""
    import torch
    stream = torch.cuda.Stream()
    handle = stream.cuda_stream
    with torch.cuda.stream(stream):
        for i in range(warmup):
            st = launch(i, handle)
            if st:
                raise RuntimeError(f"launch failed with status {st}")
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    if mode == "graph":
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(steps):
                launch(warmup + i, handle)
        torch.cuda.synchronize()
        graph.replay()  # untimed replay: graph upload
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            start.record(stream)
            graph.replay()
            end.record(stream)
        torch.cuda.synchronize()
        del graph
    else:
        with torch.cuda.stream(stream):
            start.record(stream)
            for i in range(steps):
                launch(warmup + i, handle)
            end.record(stream)
        torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3


def single_launch_median(launch, n: int, warmup: int) -> float:
    """Median seconds of single launches, each bracketed by its own pair of HIP
    events on the launch stream (eager launches; a cross-check of the per-launch
    average with the kernel durations rocprofv3 reports)."""
    import torch
    stream = torch.cuda.Stream()
    handle = stream.cuda_stream
    with torch.cuda.stream(stream):
        for i in range(warmup):
            launch(i, handle)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    with torch.cuda.stream(stream):
        for i, (a, b) in enumerate(ev):
            a.record(stream)
            st = launch(warmup + i, handle)
            b.record(stream)
            if st:
                raise RuntimeError(f"launch failed with status {st}")
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev])) / 1e3


def copy_ceiling(nbytes_rw: int, rotate_bytes: int, steps: int, warmup: int, mode="graph",
                 kind="stream"):
    """GB/s of a plain device copy moving the same bytes (read n/2, write n/2):
    kind "stream" is the library's non-temporal streaming copy (the attainable
    rate for the fused kernels' access pattern), "torch" is torch's copy_."""
    import torch
    n = nbytes_rw // 4  # bf16 elements per direction
    nsets = max(2, -(-rotate_bytes // nbytes_rw))
    src = [torch.empty(n, dtype=torch.bfloat16, device="cuda").fill_(1.0) for _ in range(nsets)]
    dst = [torch.empty_like(src[0]) for _ in range(nsets)]
    if kind == "stream":
        import diffusion_dit_adaln_amd as A
        lib = A.load_library()
        nb = n * 2

        def launch(i, h):
            return lib.adaln_diag_stream_copy(src[i % nsets].data_ptr(), dst[i % nsets].data_ptr(),
                                              nb, h)
    else:
        def launch(i, _h):
            dst[i % nsets].copy_(src[i % nsets])
            return 0

    t = time_steps(launch, steps, warmup, mode)
    return nbytes_rw * steps / t / 1e9


def stream_rate(kind: str, nbytes: int, per: int, rotate_bytes: int, steps: int,
                warmup: int) -> float:
    """GB/s of the library's streaming kernel `kind` moving `nbytes` bytes in total:
    copy reads nbytes/2 and writes nbytes/2 (a fused kernel's mix), read reads nbytes,
    fill writes nbytes.  Buffer sets rotate over >= rotate_bytes, graph replay."""
    import torch
    import diffusion_dit_adaln_amd as A
    lib = A.load_library()
    kid = {"copy": 0, "read": 1, "fill": 2}[kind]
    span = nbytes // 2 if kind == "copy" else nbytes
    span -= span % 16
    nsets = max(2, -(-rotate_bytes // nbytes))
    src = ([torch.empty(span, dtype=torch.uint8, device="cuda").fill_(1) for _ in range(nsets)]
           if kind != "fill" else [None] * nsets)
    if kind == "read":
        dst = [torch.empty(span, dtype=torch.uint8, device="cuda")] * nsets  # only the folds
    else:
        dst = [torch.empty(span, dtype=torch.uint8, device="cuda") for _ in range(nsets)]

    def launch(i, h):
        s_ = src[i % nsets]
        return lib.adaln_diag_stream(kid, None if s_ is None else s_.data_ptr(),
                                     dst[i % nsets].data_ptr(), span, per, h)

    t = time_steps(launch, steps, warmup, "graph")
    moved = 2 * span if kind == "copy" else span
    del src, dst
    torch.cuda.empty_cache()
    return moved * steps / t / 1e9


def ceilings_at(nbytes: int, rotate_bytes: int, steps: int, warmup: int, pers=STREAM_PERS):
    """The measured streaming ceilings at one byte count: for copy, read-only and
    write-only, the rate at each vector count per thread and the best of them."""
    out = {}
    for kind in ("copy", "read", "fill"):
        rates = {str(p): round(stream_rate(kind, nbytes, p, rotate_bytes, steps, warmup), 1)
                 for p in pers}
        best = max(rates, key=lambda k: rates[k])
        out[kind] = {"GBps": rates[best], "per_thread": int(best), "by_per_thread": rates}
    return out


def load_profile_table(name: str, key_col: int, val_col: int):
    """{workload: value} from a committed profile summary whose rows are
    'workload | ... | value' (columns by index), or {} when the summary is missing or
    was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return {}
    rows, sha = {}, None
    with open(path) as fh:
        for line in fh:
            if line.startswith("#"):
                if "kernel_src_sha" in line and "=" in line:
                    sha = line.split("=", 1)[1].strip()
                continue
            parts = [c.strip() for c in line.split("|")]
            if len(parts) > max(key_col, val_col):
                try:
                    rows[parts[key_col]] = float(parts[val_col])
                except ValueError:
                    pass
    return rows if sha == kernel_src_sha() else {}


def median3(f):
    v = sorted(f() for _ in range(3))
    return v[1]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s: float, y_gpu=None):
    """The C oracle, single-threaded, pinned to one core of this host, timed on the
    whole workload for about budget_s seconds.  Its output is also compared with the
    GPU's output of the same inputs (y_gpu, bf16 bits) when given."""
    from oracle import oracle as O
    affinity = sorted(os.sched_getaffinity(0))
    os.sched_setaffinity(0, {affinity[0]})
    fn = {"ln": lambda: O.layernorm_modulate(wl.x, wl.scale, wl.shift, wl.eps),
          "rms": lambda: O.rmsnorm_scale_shift(wl.x, wl.weight, wl.scale, wl.shift, wl.eps),
          "rg": lambda: O.residual_gate_rmsnorm_scale_shift(wl.res, wl.x, wl.gate, wl.weight,
                                                            wl.scale, wl.shift, wl.eps),
          "rgln": lambda: O.residual_gate_layernorm_modulate(wl.res, wl.x, wl.gate, wl.scale,
                                                             wl.shift, wl.eps),
          "lnq": lambda: O.layernorm_modulate_fp8(wl.x, wl.scale, wl.shift, wl.qscale,
                                                  wl.eps),
          "qk": lambda: O.qk_rmsnorm_rope(wl.q, wl.k, wl.q_weight, wl.k_weight, wl.cos_sin,
                                          wl.eps),
          "cf": lambda: O.residual_gate_channel_first(wl.res, wl.update, wl.gate)}[wl.op]
    # the same oracle call on a slice of rows [lo, hi) of the flattened B*T rows
    # (fused ops, one batch entry: B == 1), for the all-cores run below
    fn_rows = None
    if wl.op in ("ln", "rms", "rg", "rgln", "lnq") and wl.x.shape[0] == 1:
        def fn_rows(lo, hi):
            sl = slice(lo, hi)
            xs = wl.x[:, sl]
            rs = wl.res[:, sl] if wl.res is not None else None
            return {"ln": lambda: O.layernorm_modulate(xs, wl.scale, wl.shift, wl.eps),
                    "rms": lambda: O.rmsnorm_scale_shift(xs, wl.weight, wl.scale, wl.shift,
                                                         wl.eps),
                    "rg": lambda: O.residual_gate_rmsnorm_scale_shift(
                        rs, xs, wl.gate, wl.weight, wl.scale, wl.shift, wl.eps),
                    "rgln": lambda: O.residual_gate_layernorm_modulate(
                        rs, xs, wl.gate, wl.scale, wl.shift, wl.eps),
                    "lnq": lambda: O.layernorm_modulate_fp8(xs, wl.scale, wl.shift, wl.qscale,
                                                            wl.eps)}[wl.op]()
    first = fn()  # warm (page in the library and the arrays)
    reps = 0
    t0 = time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    os.sched_setaffinity(0, set(affinity))
    par = cpu_all_cores(wl, fn_rows, budget_s / 2, len(affinity), first)
    out = {"value": round(wl.algorithmic_bytes() * reps / el / 1e9, 4), "unit": "GB/s",
           "cores": 1, "kind": "oracle",
           "rows_per_s": round(workload_rows(wl) * reps / el, 1),
           "sample": f"the whole workload ({workload_rows(wl)} rows) x {reps} "
                     f"repetitions, single-threaded C oracle pinned to core {affinity[0]}, "
                     f"{el:.1f} s",
           "cpu_model": cpu_model(), "host_cores_available": len(affinity)}
    if par is not None:
        out["all_cores"] = par
    if y_gpu is not None:
        # the fused ops' y (the last of r, y); QK's (q_out, k_out); channel-first's out
        if wl.op == "qk":
            ref = list(first)
        else:
            ref = [first[-1] if isinstance(first, tuple) else first]
        out["gpu_output_equals_oracle"] = bool(
            len(ref) == len(y_gpu) and all(np.array_equal(np.asarray(g), r)
                                           for g, r in zip(y_gpu, ref)))
    return out


KERNEL_OF = {"qk": "qk_rmsnorm_rope", "cf": "residual_gate_cf"}


def workload_rows(wl) -> int:
    """Rows of a workload: B*T for the fused ops, head vectors for QK (tokens x
    (heads of Q + heads of K)), tokens (B*T) for the channel-first residual gate."""
    if wl.op == "qk":
        return wl.qkv.shape[0] * 2 * wl.qkv.shape[2]
    if wl.op == "cf":
        return wl.res.shape[0] * wl.res.shape[2]
    return wl.x.shape[0] * wl.x.shape[1]


def cpu_all_cores(wl, fn_rows, budget_s: float, cores: int, single):
    """The same oracle, rows split evenly over `cores` threads (the C oracle holds no
    shared state and ctypes releases the GIL), timed for about budget_s seconds; its
    output must equal the single-threaded one bit for bit.  None when not applicable."""
    if fn_rows is None or cores < 2:
        return None
    from concurrent.futures import ThreadPoolExecutor
    rows = wl.x.shape[1]
    cuts = [rows * i // cores for i in range(cores + 1)]
    parts = [(cuts[i], cuts[i + 1]) for i in range(cores) if cuts[i + 1] > cuts[i]]

    def last(r):
        return r[-1] if isinstance(r, tuple) else r

    with ThreadPoolExecutor(len(parts)) as pool:
        got = list(pool.map(lambda lh: last(fn_rows(*lh)), parts))
        same = bool(np.array_equal(np.concatenate(got, axis=1), last(single)))
        reps = 0
        t0 = time.perf_counter()
        while True:
            list(pool.map(lambda lh: fn_rows(*lh), parts))
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    return {"value": round(wl.algorithmic_bytes() * reps / el / 1e9, 4), "unit": "GB/s",
            "cores": len(parts), "equals_single_core": same,
            "sample": f"the whole workload x {reps}, rows split over {len(parts)} threads, "
                      f"{el:.1f} s"}


def inputs_sha256(wl) -> dict:
    """SHA-256 (first 16 hex digits) of every input buffer of a workload."""
    out = {}
    for name in ("x", "res", "scale", "shift", "gate", "weight", "qkv", "q_weight", "k_weight",
                 "cos_sin", "update"):
        a = getattr(wl, name, None)
        if a is not None:
            out[name] = hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]
    return out


def describe(wl):
    if wl.op == "qk":
        T, _, Hd, D = wl.qkv.shape
        return (f"qk_rmsnorm_rope bf16 q, k [{T},{Hd},{D}] as views of packed qkv "
                f"[{T},3,{Hd},{D}], weights 1+0.02N, fp32 cos/sin cache, eps 1e-6")
    if wl.op == "cf":
        B, H, T = wl.res.shape
        return (f"residual_gate_channel_first bf16 res/out [{B},{H},{T}], "
                f"update [{B},{T},{H}], gate [{B},{H}]")
    B, T, H = wl.x.shape
    name = {"ln": "layernorm_modulate", "rms": "rmsnorm_scale_shift",
            "rg": "residual_gate_rmsnorm_scale_shift",
            "rgln": "residual_gate_layernorm_modulate",
            "lnq": "layernorm_modulate_fp8_quant"}[wl.op]
    extra = {"rms": " weight 1+0.02N", "rg": " weight none",
             "lnq": f" -> E4M3, static scale {wl.qscale}"}.get(wl.op, "")
    return f"{name} bf16 [{B},{T},{H}]{extra}, eps 1e-6"


def sweep_rows(rotate: int, steps: int, warmup: int, op: str = "rms") -> None:
    """One JSON line: per row count, the fused kernel's (RMS at H 4096 or LayerNorm at
    H 3072) and the streaming copy's GB/s and microseconds per launch (graph replay),
    and the least-squares fit of the kernel's time per launch to fixed + bytes / rate."""
    from diffusion_dit_adaln_amd import synth
    make = synth.rms_rows if op == "rms" else synth.ln_rows
    points = []
    for T in (256, 512, 1024, 2048, 4216, 8192, 16384, 32768, 65536):
        wl = make(T)
        L = launcher_for(wl, rotate)
        nbytes = wl.algorithmic_bytes()
        t = time_steps(L.call, steps, warmup, "graph") / steps
        del L
        c = copy_ceiling(nbytes, rotate, steps, warmup)
        points.append({"rows": T, "bytes": nbytes, "GBps": round(nbytes / t / 1e9, 1),
                       "us_per_launch": round(t * 1e6, 3), "copy_GBps": round(c, 1),
                       "frac_of_copy": round(nbytes / t / 1e9 / c, 4)})
        print(f"[sweep] rows {T}: {points[-1]['GBps']} GB/s, copy {points[-1]['copy_GBps']}",
              file=sys.stderr, flush=True)
    b = np.array([p["bytes"] for p in points], dtype=np.float64)
    u = np.array([p["us_per_launch"] for p in points], dtype=np.float64)
    slope, fixed = np.polyfit(b, u, 1)
    name = ("rmsnorm_scale_shift bf16 [1,T,4096] weight" if op == "rms"
            else "layernorm_modulate bf16 [1,T,3072]")
    print(json.dumps({"sweep": name + ", graph replay",
                      "points": points,
                      "fit": {"fixed_us": round(float(fixed), 3),
                              "asymptotic_GBps": round(float(1e-3 / slope), 1)}}), flush=True)


def time_workload(name: str, rotate: int, steps: int, warmup: int, modes=("graph", "eager")):
    """Median-of-3 GB/s and microseconds per launch of one workload, per timing mode."""
    import torch
    w = workload(name)
    L = launcher_for(w, rotate)
    nb = w.algorithmic_bytes()
    res = {}
    for mode in modes:
        t = median3(lambda: time_steps(L.call, steps, warmup, mode))
        res[mode] = {"GBps": round(nb * steps / t / 1e9, 2),
                     "us_per_launch": round(t / steps * 1e6, 3)}
    del L
    torch.cuda.empty_cache()
    return w, nb, res


def config_roofline(name: str, rotate: int, steps: int, warmup: int, ceil_1g: dict):
    """The roofline object of one target configuration: the rate between HIP events
    (graph replay, median of 3), the committed kernel-trace time and traffic ratio
    (when taken on the current kernel source), and the fractions of the 8 TB/s peak
    and of the measured streaming ceilings at the same bytes and at 1 GiB."""
    w, nb, res = time_workload(name, rotate, steps, warmup)
    gbps = res["graph"]["GBps"]
    trace_ns = load_profile_table("kernel_trace_configs.txt", 0, 3).get(name)
    ratio = load_profile_table("counters_all_workloads.txt", 0, 6).get(name)
    ceil = ceilings_at(nb, rotate, steps, warmup)
    out = {"workload": describe(w), "bytes": nb, "rows": workload_rows(w),
           "bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
           "frac": round(gbps / PEAK_HBM_GBPS, 4),
           "us_per_launch": res["graph"]["us_per_launch"], "eager": res["eager"],
           "trace_us": None if trace_ns is None else round(trace_ns / 1e3, 3),
           "trace_GBps": None if trace_ns is None else round(nb / trace_ns, 1),
           "traffic_ratio": ratio,
           "traffic": None if ratio is None else round(ratio * nb),
           "ceiling": {k: {"GBps": v["GBps"], "per_thread": v["per_thread"]}
                       for k, v in ceil.items()},
           "frac_of_copy": round(gbps / ceil["copy"]["GBps"], 4),
           "frac_of_copy_1GiB": round(gbps / ceil_1g["copy"]["GBps"], 4),
           "meets_target": gbps >= TARGET_FRAC * PEAK_HBM_GBPS,
           "copy_meets_target": ceil["copy"]["GBps"] >= TARGET_FRAC * PEAK_HBM_GBPS}
    if trace_ns is not None:
        out["trace_frac"] = round(nb / trace_ns / PEAK_HBM_GBPS, 4)
    return out, ceil


CF_SWEEP_TOKENS = (4608, 4336, 4333, 4334, 4332, 4335)


def sweep_cf(rotate: int, steps: int, warmup: int) -> None:
    """One JSON line: the channel-first residual gate at [2, 3072, T] for token counts
    T with every residue of T mod 8 that matters (0: aligned rows; odd, 2 and 4 mod 8:
    rows starting inside a 16-byte block), GB/s per launch in graph replay (median of
    3) beside the best streaming copy of the same bytes."""
    from diffusion_dit_adaln_amd import synth
    points = []
    for T in CF_SWEEP_TOKENS:
        wl = synth.cf_tokens(T)
        L = launcher_for(wl, rotate)
        nb = wl.algorithmic_bytes()
        t = median3(lambda: time_steps(L.call, steps, warmup, "graph")) / steps
        del L
        cc = max(stream_rate("copy", nb, p, rotate, steps, warmup) for p in (1, 4, 8))
        points.append({"tokens": T, "T_mod_8": T % 8, "bytes": nb,
                       "GBps": round(nb / t / 1e9, 1), "us_per_launch": round(t * 1e6, 3),
                       "copy_GBps": round(cc, 1), "frac_of_copy": round(nb / t / 1e9 / cc, 4)})
        print(f"[sweep-cf] T={T}: {points[-1]['GBps']} GB/s", file=sys.stderr, flush=True)
    base = next(p["GBps"] for p in points if p["tokens"] == 4336)
    for p in points:
        p["rate_vs_T4336"] = round(p["GBps"] / base, 4)
    print(json.dumps({"sweep": "residual_gate_channel_first bf16 res/out [2,3072,T], "
                               "update [2,T,3072], graph replay", "points": points}), flush=True)


def all_workloads(rotate: int, steps: int, warmup: int, mode: str) -> None:
    """For profiler runs: every workload (and the channel-first sweep's token counts)
    launched `steps` times after `warmup`, then the library's streaming copy (8
    vectors per thread) of the same byte count `steps` times; one JSON line per
    workload, in this order, so that a trace or counter file can be split by it."""
    import torch
    from diffusion_dit_adaln_amd import synth
    names = WORKLOAD_NAMES + [f"cf:{T}" for T in CF_SWEEP_TOKENS if T != 4608]
    for name in names:
        wl = synth.cf_tokens(int(name[3:])) if name.startswith("cf:") else workload(name)
        L = launcher_for(wl, rotate)
        nb = wl.algorithmic_bytes()
        t = time_steps(L.call, steps, warmup, mode)
        del L
        torch.cuda.empty_cache()
        c = copy_ceiling(nb, rotate, steps, warmup, mode)
        print(json.dumps({"workload": wl.name, "op": wl.op, "bytes": nb,
                          "GBps": round(nb * steps / t / 1e9, 2),
                          "copy_GBps": round(c, 2)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default=HEADLINE, choices=WORKLOAD_NAMES,
                    help="the workload of the timed line (default: LayerNorm [2,4608,3072])")
    ap.add_argument("--timing", default="graph", choices=["graph", "eager"])
    ap.add_argument("--rotate-mb", type=int, default=1024)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed workload (for profiler runs)")
    ap.add_argument("--sweep-rows", action="store_true",
                    help="instead of the benchmark line: one op (--sweep-op) over a range of "
                         "row counts beside the streaming copy of the same bytes, with a fit "
                         "of time = fixed + bytes / rate")
    ap.add_argument("--sweep-op", default="rms", choices=["rms", "ln"],
                    help="the op of --sweep-rows: RMS at H 4096 or LayerNorm at H 3072")
    ap.add_argument("--sweep-cf", action="store_true",
                    help="instead of the benchmark line: the channel-first residual gate over "
                         "token counts with aligned and unaligned residual rows")
    ap.add_argument("--cf-tokens", type=int, default=0,
                    help="with --workload rg_channel_first_2x3072x4608: use this token count "
                         "instead (for profiler runs of the sweep's shapes)")
    ap.add_argument("--copy-only", action="store_true",
                    help="only a plain device copy of the workload's byte count (counter "
                         "calibration for profiler runs)")
    ap.add_argument("--all-workloads", action="store_true",
                    help="instead of the benchmark line: every workload and a same-bytes "
                         "copy, --steps launches each (for profiler runs)")
    ap.add_argument("--ceilings", action="store_true",
                    help="instead of the benchmark line: the streaming ceilings (copy, "
                         "read-only, write-only, 1..16 vectors per thread) at each target "
                         "configuration's bytes and at 1 GiB")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this path runs on one GPU; row-sharding it across GPUs needs no "
              "collective and is not measured here (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)

    rotate = args.rotate_mb << 20
    if args.sweep_rows:
        sweep_rows(rotate, args.steps, args.warmup, args.sweep_op)
        return
    if args.all_workloads:
        all_workloads(rotate, args.steps, args.warmup, args.timing)
        return
    if args.sweep_cf:
        sweep_cf(rotate, args.steps, args.warmup)
        return
    if args.ceilings:
        table = {}
        for name in TARGET_CONFIGS + ["1GiB"]:
            nb = (1 << 30) if name == "1GiB" else workload(name).algorithmic_bytes()
            table[name] = {"bytes": nb, **ceilings_at(nb, rotate, max(50, args.steps // 4),
                                                      args.warmup)}
            print(f"[ceilings] {name} done", file=sys.stderr, flush=True)
        print(json.dumps({"ceilings": table}), flush=True)
        return
    wl = workload(args.workload)
    if args.cf_tokens:
        if wl.op != "cf":
            ap.error("--cf-tokens applies to the channel-first workload")
        from diffusion_dit_adaln_amd import synth
        wl = synth.cf_tokens(args.cf_tokens)
    if args.copy_only:
        g = copy_ceiling(wl.algorithmic_bytes(), rotate, args.steps, args.warmup, args.timing)
        # (the library's streaming copy kernel, 8 vectors per thread: known bytes for
        # counter scaling)
        print(json.dumps({"copy_GBps": round(g, 2), "bytes_per_copy": wl.algorithmic_bytes(),
                          "read_bytes": wl.algorithmic_bytes() // 2,
                          "write_bytes": wl.algorithmic_bytes() // 2}), flush=True)
        return
    L = launcher_for(wl, rotate)
    nbytes = wl.algorithmic_bytes()
    rows = workload_rows(wl)

    t = time_steps(L.call, args.steps, args.warmup, args.timing)
    gbps = nbytes * args.steps / t / 1e9

    # the outputs of buffer set 0 (every set holds the same inputs), as bits
    def bits(t):
        return t.cpu().numpy() if t.dtype == torch.uint8 else \
            t.cpu().view(torch.int16).numpy().view(np.uint16)
    s0 = L.sets[0]
    y_gpu = [bits(s0[k]) for k in ("y", "qo", "ko", "out") if k in s0]
    ms_per_step = t / args.steps * 1e3
    # average launch duration of the fused kernel: the same events, per launch
    avg_launch_s = t / args.steps

    traffic = load_counters(wl.name)
    if traffic is None:
        ratio = load_profile_table("counters_all_workloads.txt", 0, 6).get(wl.name)
        traffic = None if ratio is None else round(ratio * nbytes)
    out = {
        "metric": METRIC, "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": describe(wl), "io_dtype": "bf16", "rows": rows,
                   "bytes_per_step": nbytes, "rotation_sets": L.nsets, "timing": args.timing,
                   "inputs_sha256": inputs_sha256(wl)},
        "pct_of_peak": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
        "rows_per_s": round(rows * args.steps / t, 1),
        "roofline": {"bound": "hbm", "achieved": round(nbytes / avg_launch_s / 1e9, 2),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(nbytes / avg_launch_s / 1e9 / PEAK_HBM_GBPS, 4),
                     "traffic": traffic,
                     "kernel": KERNEL_OF.get(wl.op, f"fused_norm_modulate ({wl.op})"),
                     "avg_launch_us": round(avg_launch_s * 1e6, 3)},
    }
    # per-launch cross-check: median of single launches between their own events
    med = single_launch_median(L.call, 200, args.warmup)
    out["roofline"]["single_launch_median_us"] = round(med * 1e6, 3)
    out["roofline"]["single_launch_median_GBps"] = round(nbytes / med / 1e9, 2)
    trace_ns = load_profile_table("kernel_trace_configs.txt", 0, 3).get(wl.name)
    if trace_ns is not None:
        out["roofline"]["trace_us"] = round(trace_ns / 1e3, 3)
    del L
    torch.cuda.empty_cache()
    if not args.no_extras:
        steps = max(50, args.steps // 2)
        ceil_1g = ceilings_at(1 << 30, rotate, steps // 2, args.warmup)
        out["ceilings_1GiB"] = ceil_1g
        per_config = {}
        for name in TARGET_CONFIGS:
            per_config[name], _ = config_roofline(name, rotate, steps, args.warmup, ceil_1g)
            print(f"[bench] {name} done", file=sys.stderr, flush=True)
        out["per_config"] = per_config
        if wl.name in per_config:
            pc = per_config[wl.name]
            out["roofline"]["frac_of_copy"] = round(gbps / pc["ceiling"]["copy"]["GBps"], 4)
            out["roofline"]["ceiling"] = pc["ceiling"]
        out["configs_meeting_target"] = sum(1 for v in per_config.values() if v["meets_target"])
        per = {}
        for name in WORKLOAD_NAMES:
            if name in TARGET_CONFIGS:
                continue
            w2, nb2, res = time_workload(name, rotate, steps, args.warmup)
            cc = max(stream_rate("copy", nb2, p, rotate, steps, args.warmup) for p in (4, 8, 16))
            shape = list({"qk": lambda: w2.qkv.shape, "cf": lambda: w2.res.shape}.get(
                w2.op, lambda: w2.x.shape)())
            per[w2.name] = {"op": w2.op, "shape": shape, "bytes": nb2, **res,
                            "rows_per_s": round(workload_rows(w2) / res["graph"]["us_per_launch"]
                                                * 1e6, 1),
                            "frac_of_peak": round(res["graph"]["GBps"] / PEAK_HBM_GBPS, 4),
                            "copy_ceiling_GBps": round(cc, 2),
                            "frac_of_copy_ceiling": round(res["graph"]["GBps"] / cc, 4)}
            print(f"[bench] {name} done", file=sys.stderr, flush=True)
        out["per_workload"] = per
    if not args.no_cpu:
        cb = cpu_baseline(wl, args.cpu_seconds, y_gpu=y_gpu)
        cb["cores"] = 1
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
