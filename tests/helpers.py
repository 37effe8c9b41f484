"""Shared helpers for the GPU tests (host <-> device bf16 bit patterns)."""
import sys

import numpy as np
import torch


def say(*a):
    """Name the case before GPU work, flushed, so a lost run still tells what ran."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a, device="cuda"):
    """numpy uint16 bf16 bits -> device bfloat16 tensor (same shape)."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)


def host(t):
    """device/host bfloat16 tensor -> numpy uint16 bits."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def first_diff(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    idx = np.argwhere(a != b)
    if len(idx) == 0:
        return None
    i = tuple(idx[0])
    return f"{len(idx)} differing elements; first at {i}: got 0x{int(a[i]):04x} want 0x{int(b[i]):04x}"


def assert_bits_equal(got, want, what=""):
    d = first_diff(got, want)
    assert d is None, f"{what}: {d}"
