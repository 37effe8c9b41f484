"""Exhaustive pins of the oracle's rounding primitives (CPU).

Every binary32 input of the bf16 rounding, and every pair of bf16 operands of the
two binary32 operations the modulate and residual-gate chains are built from
(product and sum, each rounded to binary32 and then to bf16), checked against
references that share nothing with the oracle:

  * the bf16 rounding against torch's float32 -> bfloat16 conversion;
  * products and sums against numpy float64 arithmetic followed by the correctly
    rounded float64 -> float32 conversion and torch's bfloat16 conversion.  A product
    of two bf16 values (8-bit significands) is exact in float64.  A sum is exact in
    float64 unless the exponents differ by more than 45, and then the smaller operand
    is far below half a binary32 ulp of the larger, so the float32 result is still the
    correctly rounded one.

The oracle's product is reached as round(-0 + round(gate * x)) (adding -0 changes no
value, -0 included) and its sum as round(res + round(1 * x)) (x is a bf16 value).
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import oracle as O

ALL16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
BLOCK = 64  # first operands per chunk: 64 x 65536 pairs
WORKERS = 8


def _rb(f32):
    """binary32 -> bf16 bits by torch's conversion."""
    t = torch.from_numpy(np.ascontiguousarray(f32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _same(got, ref):
    """Bitwise equal, except that NaN must meet NaN (payloads are not compared)."""
    gn = (got & 0x7F80) == 0x7F80
    gn &= (got & 0x007F) != 0
    rn = (ref & 0x7F80) == 0x7F80
    rn &= (ref & 0x007F) != 0
    return np.array_equal(gn, rn) and np.array_equal(got[~rn], ref[~rn])


def _pairs(i):
    a = np.repeat(ALL16[i * BLOCK:(i + 1) * BLOCK], 1 << 16)
    b = np.tile(ALL16, BLOCK)
    return a, b


def _run(check):
    threads = torch.get_num_threads()
    torch.set_num_threads(1)  # parallel over chunks instead
    try:
        def quiet(i):  # overflow to inf and inf - inf are expected (numpy's state is per thread)
            with np.errstate(over="ignore", invalid="ignore"):
                return check(i)
        with ThreadPoolExecutor(WORKERS) as pool:
            bad = [i for i, ok in enumerate(pool.map(quiet, range((1 << 16) // BLOCK))) if not ok]
    finally:
        torch.set_num_threads(threads)
    assert not bad, f"chunks with mismatches: {bad[:8]}"


def test_bf16_rounding_all_binary32_inputs():
    def check(i):
        u = (np.arange(i * BLOCK, (i + 1) * BLOCK, dtype=np.uint32)[:, None] << 16
             | np.arange(1 << 16, dtype=np.uint32)[None, :]).reshape(-1)
        x = u.view(np.float32)
        got = O.round_bf16(x)
        ref = _rb(x)
        ok = _same(got, ref)
        # a NaN keeps its sign
        nan = np.isnan(x)
        return ok and np.array_equal(got[nan] >> 15, (u[nan] >> 31).astype(np.uint16))
    _run(check)


def test_products_all_bf16_pairs():
    minus_zero = np.full(BLOCK << 16, 0x8000, np.uint16)

    def check(i):
        a, b = _pairs(i)
        got = O.gate_residual(minus_zero, b, a)             # round(-0 + round(a*b))
        ref = _rb((_f64(a) * _f64(b)).astype(np.float32))
        return _same(got, ref)
    _run(check)


def test_sums_all_bf16_pairs():
    one = np.full(BLOCK << 16, 0x3F80, np.uint16)

    def check(i):
        a, b = _pairs(i)
        got = O.gate_residual(a, b, one)                    # round(a + round(1*b))
        ref = _rb((_f64(a) + _f64(b)).astype(np.float32))
        return _same(got, ref)
    _run(check)


# --------------------------------------------------------------------------
# brute force over the two exhaustive row domains (tests/brute_domains.py)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["h8", "h16"])
def test_brute_force_full_domains(name):
    """Every row of 8 values over {0, +-0.5, +-1, +-2, 3} and of 16 values over
    {-1, 0, 1}: the oracle's LayerNorm and RMSNorm outputs lie within 2 bf16 ulp of
    the float64 definition (with the LayerNorm floor of the mean's own error), and
    its modulated outputs hash to the digests stored in tests/golden, which the GPU
    test compares the device's outputs with.  Worker processes, no GPU."""
    from tests import brute_domains as D

    d_ln, d_rms, bad = D.oracle_digests(name, check=True)
    assert bad == 0, f"{bad} norm outputs outside the float64 bound"
    g = D.golden_digests()
    assert (d_ln, d_rms) == (g[(name, "ln")], g[(name, "rms")])

