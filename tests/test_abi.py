"""The C-ABI library loads, exports every symbol include/adaln.h declares, agrees
with the oracle on the reduction layout, and rejects bad arguments before any GPU
work (no compute call is made here, so these run without a GPU)."""
import os
import re

import pytest

import diffusion_dit_adaln_amd as A
from diffusion_dit_adaln_amd import _binding
from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "adaln.h")

OK, NULL, SHAPE, ALIGN, STRIDE, OVERLAP, VALUE, LAUNCH = range(8)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(A.library_path()):
        pytest.fail("libadaln.so is not built: run python __graft_entry__.py")
    return A.load_library()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(adaln_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_are_exported(lib):
    names = declared_symbols()
    assert len(names) == 24, names
    assert set(names) == set(_binding.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings(lib):
    assert A.adaln_abi_version() == A.ABI_VERSION == 11
    for s in range(8):
        assert len(A.adaln_status_string(s)) > 5
    assert A.adaln_status_string(99) == "unknown status"


def test_layout_matches_oracle_for_every_h(lib):
    for H in range(8, 8193, 8):
        assert A.adaln_reduction_layout(H) == O.layout(H), H
    for H in [0, 4, 12, 8200, -8]:
        with pytest.raises(A.AdalnError):
            A.adaln_reduction_layout(H)


# fake, well-separated, 16-byte aligned "device" addresses: validation never
# dereferences them
BASE = 1 << 40


def addr(i):
    return BASE + i * (1 << 34)


def ln_args(**kw):
    a = dict(x=addr(0), scale=addr(1), shift=addr(2), y=addr(3), B=2, T=5, H=3072, sbs=3072,
             hbs=3072, eps=1e-6)
    a.update(kw)
    return a


def ln_check(lib, **kw):
    a = ln_args(**kw)
    return lib.adaln_check_layernorm_modulate(a["x"], a["scale"], a["shift"], a["y"], a["B"],
                                              a["T"], a["H"], a["sbs"], a["hbs"], a["eps"])


def rg_check(lib, **kw):
    a = dict(res=addr(0), x=addr(1), gate=addr(2), w=addr(3), scale=addr(4), shift=addr(5),
             r=addr(6), y=addr(7), B=2, T=5, H=4096, gbs=4096, sbs=4096, hbs=4096, eps=1e-6)
    a.update(kw)
    return lib.adaln_check_residual_gate_rmsnorm_scale_shift(
        a["res"], a["x"], a["gate"], a["w"], a["scale"], a["shift"], a["r"], a["y"], a["B"],
        a["T"], a["H"], a["gbs"], a["sbs"], a["hbs"], a["eps"])


def rgln_check(lib, **kw):
    a = dict(res=addr(0), x=addr(1), gate=addr(2), scale=addr(4), shift=addr(5), r=addr(6),
             y=addr(7), B=2, T=5, H=3072, gbs=3072, sbs=3072, hbs=3072, eps=1e-6)
    a.update(kw)
    return lib.adaln_check_residual_gate_layernorm_modulate(
        a["res"], a["x"], a["gate"], a["scale"], a["shift"], a["r"], a["y"], a["B"], a["T"],
        a["H"], a["gbs"], a["sbs"], a["hbs"], a["eps"])


def lnq_check(lib, **kw):
    a = dict(x=addr(0), scale=addr(1), shift=addr(2), qs=addr(3), q=addr(4), B=2, T=5, H=3072,
             sbs=3072, hbs=3072, eps=1e-6)
    a.update(kw)
    return lib.adaln_check_layernorm_modulate_fp8_quant(a["x"], a["scale"], a["shift"], a["qs"],
                                                        a["q"], a["B"], a["T"], a["H"], a["sbs"],
                                                        a["hbs"], a["eps"])


def test_fp8_quant_checks(lib):
    assert lnq_check(lib) == OK
    assert lnq_check(lib, qs=None) == NULL
    assert lnq_check(lib, q=None) == NULL
    assert lnq_check(lib, qs=addr(3) + 2) == ALIGN
    assert lnq_check(lib, qs=addr(3) + 4) == OK          # 4-byte alignment suffices
    assert lnq_check(lib, q=addr(4) + 8) == ALIGN
    assert lnq_check(lib, H=12) == SHAPE
    rows_bytes = 2 * 5 * 3072                            # one byte per element
    assert lnq_check(lib, q=addr(0) + 2 * rows_bytes) == OK      # just after x (2 bytes/elem)
    assert lnq_check(lib, q=addr(0) + 2 * rows_bytes - 16) == OVERLAP
    assert lnq_check(lib, qs=addr(4) + rows_bytes - 4) == OVERLAP  # scale inside q
    assert lnq_check(lib, qs=addr(4) + rows_bytes) == OK
    assert lnq_check(lib, B=0, x=None, q=None, qs=None) == OK
    assert lib.adaln_layernorm_modulate_fp8_quant(addr(0), addr(1), addr(2), None, addr(4), 1, 2,
                                                  3072, 0, 0, 1e-6, None) == NULL
    assert lib.adaln_diag_quant_fp8(addr(0), addr(1), 6, addr(2), None) == SHAPE
    assert lib.adaln_diag_quant_fp8(addr(0) + 4, addr(1), 8, addr(2), None) == ALIGN
    assert lib.adaln_diag_quant_fp8(addr(0), addr(0) + 8, 8, addr(2), None) == OVERLAP
    assert lib.adaln_diag_quant_fp8(None, None, 0, None, None) == OK


def qk_check(lib, **kw):
    a = dict(q=addr(0), k=addr(0) + 3072 * 2, wq=addr(1), wk=addr(2), cs=addr(3), qo=addr(4),
             ko=addr(5), T=7, hq=24, hk=24, D=128, qts=3 * 3072, kts=3 * 3072, eps=1e-6)
    a.update(kw)
    return lib.adaln_check_qk_rmsnorm_rope(a["q"], a["k"], a["wq"], a["wk"], a["cs"], a["qo"],
                                           a["ko"], a["T"], a["hq"], a["hk"], a["D"], a["qts"],
                                           a["kts"], a["eps"])


def test_qk_checks(lib):
    assert qk_check(lib) == OK                          # packed QKV views
    assert qk_check(lib, wq=None, wk=None) == OK
    assert qk_check(lib, D=64) == SHAPE
    assert qk_check(lib, hq=-1) == SHAPE
    assert qk_check(lib, T=0, q=None, k=None, cs=None, qo=None, ko=None) == OK
    assert qk_check(lib, hk=0, k=None, ko=None) == OK
    assert qk_check(lib, cs=None) == NULL
    assert qk_check(lib, ko=None) == NULL
    assert qk_check(lib, q=addr(0) + 8) == ALIGN
    assert qk_check(lib, cs=addr(3) + 4) == ALIGN
    assert qk_check(lib, qts=3072 * 2 - 8) == OK         # any stride >= heads_q*128, % 8
    assert qk_check(lib, qts=3000) == STRIDE             # < heads_q*128
    assert qk_check(lib, kts=3 * 3072 + 4) == STRIDE     # not % 8
    assert qk_check(lib, T=1, qts=0, kts=0) == OK        # stride unused for one token
    assert qk_check(lib, eps=float("nan")) == VALUE
    # a token's heads are addressed with 32-bit byte offsets: at most 2^23 - 8 heads
    big = (1 << 23) - 8
    assert qk_check(lib, T=1, hq=big, hk=0, k=None, ko=None, qts=0) == OK
    assert qk_check(lib, T=1, hq=big + 1, hk=0, k=None, ko=None, qts=0) == SHAPE
    assert qk_check(lib, T=1, hq=0, hk=big + 1, q=None, qo=None, kts=0) == SHAPE
    assert qk_check(lib, qo=addr(0)) == OVERLAP          # output over the packed input
    assert qk_check(lib, ko=addr(4) + 16) == OVERLAP     # q_out and k_out overlap
    assert qk_check(lib, qo=addr(3) - 16) == OVERLAP     # runs into the cache
    assert lib.adaln_qk_rmsnorm_rope(addr(0), addr(1), None, None, addr(3), addr(4), addr(5), 7,
                                     24, 24, 96, 3072, 3072, 1e-6, None) == SHAPE


def cf_check(lib, **kw):
    a = dict(res=addr(0), upd=addr(1), gate=addr(2), out=addr(3), B=2, T=4608, H=3072,
             gbs=3072)
    a.update(kw)
    return lib.adaln_check_residual_gate_channel_first(a["res"], a["upd"], a["gate"], a["out"],
                                                       a["B"], a["T"], a["H"], a["gbs"])


def test_channel_first_checks(lib):
    assert cf_check(lib) == OK
    assert cf_check(lib, out=addr(0)) == OK              # in place
    assert cf_check(lib, out=addr(0) + 16) == OVERLAP    # partial overlap with res
    assert cf_check(lib, out=addr(1)) == OVERLAP         # over update
    assert cf_check(lib, T=4333) == OK                   # ragged token count
    assert cf_check(lib, H=12) == SHAPE
    # one tile per workgroup of 256, the grid rounded up to a multiple of eight
    # workgroups, fewer than 2^32 work-items: at most 2^24 - 8 tiles
    assert cf_check(lib, B=(1 << 24) - 8, T=64, H=8, gbs=0) == OK
    assert cf_check(lib, B=(1 << 24) - 7, T=64, H=8, gbs=0) == SHAPE
    # T % 64 != 0: a row's tiles start on a 128-byte line and cover T + 63 tokens
    assert cf_check(lib, B=(1 << 23) - 4, T=8, H=8, gbs=0) == OK      # two tiles each
    assert cf_check(lib, B=(1 << 23) - 3, T=8, H=8, gbs=0) == SHAPE
    far_r = dict(res=addr(0), upd=addr(10), out=addr(20), gate=addr(30), gbs=0, T=4333)
    assert cf_check(lib, B=5065, **far_r) == OK          # 48 * 69 tiles per batch entry
    assert cf_check(lib, B=5066, **far_r) == SHAPE
    far = dict(res=addr(0), upd=addr(10), out=addr(20), gate=addr(30), gbs=0)  # 137 GB each
    assert cf_check(lib, B=4854, **far) == OK            # 4854 * 48 * 72 tiles
    assert cf_check(lib, B=4855, **far) == SHAPE
    assert cf_check(lib, B=0, res=None, upd=None, gate=None, out=None) == OK
    assert cf_check(lib, upd=None) == NULL
    assert cf_check(lib, gate=None) == NULL
    assert cf_check(lib, res=addr(0) + 2) == ALIGN
    assert cf_check(lib, gbs=100) == STRIDE
    assert cf_check(lib, gbs=0) == OK
    assert lib.adaln_residual_gate_channel_first(addr(0), addr(1), addr(2), addr(1), 2, 4608,
                                                 3072, 3072, None) == OVERLAP


def test_valid_arguments_pass(lib):
    assert ln_check(lib) == OK
    assert rg_check(lib) == OK
    assert rg_check(lib, w=None) == OK
    assert rgln_check(lib) == OK
    assert rgln_check(lib, gbs=6 * 3072, sbs=6 * 3072, hbs=6 * 3072) == OK
    assert lib.adaln_check_rmsnorm_scale_shift(addr(0), None, addr(1), addr(2), addr(3), 1, 7,
                                               2048, 0, 0, 1e-6) == OK
    # FLUX chunk views: scale/shift are slices of one [B, 6H] embedding
    assert ln_check(lib, scale=addr(1) + 2 * 3072, shift=addr(1), sbs=6 * 3072, hbs=6 * 3072) == OK
    assert ln_check(lib, sbs=0, hbs=0) == OK           # one vector shared by the batch
    assert ln_check(lib, B=1, sbs=5, hbs=-3) == OK     # stride unused when B == 1


def test_empty_is_a_noop(lib):
    assert ln_check(lib, B=0, x=None, y=None, scale=None, shift=None) == OK
    assert ln_check(lib, T=0, x=None) == OK
    # the compute entry point also returns before touching anything
    assert lib.adaln_layernorm_modulate(None, None, None, None, 0, 3, 3072, 0, 0, 1e-6, None) == OK


@pytest.mark.parametrize("H", [0, 4, 12, 8200, 8193, -8, 1 << 20])
def test_bad_h(lib, H):
    assert ln_check(lib, H=H) == SHAPE


def test_bad_sizes(lib):
    assert ln_check(lib, B=-1) == SHAPE
    assert ln_check(lib, T=-2) == SHAPE
    assert ln_check(lib, B=1 << 40, T=1 << 40) == SHAPE


def test_nulls(lib):
    assert ln_check(lib, x=None) == NULL
    assert ln_check(lib, y=None) == NULL
    assert ln_check(lib, scale=None) == NULL
    assert ln_check(lib, shift=None) == NULL
    assert rg_check(lib, res=None) == NULL
    assert rg_check(lib, gate=None) == NULL
    assert rg_check(lib, r=None) == NULL
    assert rgln_check(lib, res=None) == NULL
    assert rgln_check(lib, gate=None) == NULL
    assert rgln_check(lib, r=None) == NULL
    assert rgln_check(lib, scale=None) == NULL


def test_alignment(lib):
    assert ln_check(lib, x=addr(0) + 2) == ALIGN
    assert ln_check(lib, y=addr(3) + 8) == ALIGN
    assert ln_check(lib, scale=addr(1) + 2) == ALIGN
    assert rg_check(lib, w=addr(3) + 4) == ALIGN
    assert rg_check(lib, r=addr(6) + 2) == ALIGN
    assert rgln_check(lib, res=addr(0) + 8) == ALIGN
    assert rgln_check(lib, gate=addr(2) + 2) == ALIGN


def test_strides(lib):
    assert ln_check(lib, sbs=-8) == STRIDE
    assert ln_check(lib, sbs=3076) == STRIDE      # not a multiple of 8
    assert ln_check(lib, hbs=1024) == STRIDE      # in (0, H)
    assert rg_check(lib, gbs=8) == STRIDE
    assert rgln_check(lib, gbs=3072 + 4) == STRIDE
    assert rgln_check(lib, H=3068) == SHAPE
    assert rgln_check(lib, eps=-1.0) == VALUE


def test_eps(lib):
    assert ln_check(lib, eps=-1e-6) == VALUE
    assert ln_check(lib, eps=float("nan")) == VALUE
    assert ln_check(lib, eps=float("inf")) == VALUE


def test_overlaps(lib):
    rows_bytes = 2 * 5 * 3072 * 2
    assert ln_check(lib, y=addr(0)) == OVERLAP                      # y == x
    assert ln_check(lib, y=addr(0) + rows_bytes - 16) == OVERLAP    # tail of x
    assert ln_check(lib, y=addr(0) + rows_bytes) == OK              # just after x
    assert ln_check(lib, y=addr(1) - 16) == OVERLAP                 # runs into scale
    assert rg_check(lib, r=addr(7)) == OVERLAP                      # r == y
    assert rg_check(lib, r=addr(0)) == OVERLAP                      # r == res
    assert rg_check(lib, y=addr(2)) == OVERLAP                      # y over gate
    assert rg_check(lib, y=addr(3)) == OVERLAP                      # y over weight
    assert rgln_check(lib, r=addr(7)) == OVERLAP                    # r == y
    assert rgln_check(lib, y=addr(1)) == OVERLAP                    # y over x
    assert rgln_check(lib, r=addr(2)) == OVERLAP                    # r over gate


def test_compute_entry_points_reject_before_launch(lib):
    # invalid calls return their status without any HIP call (no GPU here)
    assert lib.adaln_layernorm_modulate(addr(0), addr(1), addr(2), addr(0), 1, 2, 3072, 0, 0,
                                        1e-6, None) == OVERLAP
    assert lib.adaln_rmsnorm_scale_shift(addr(0), None, addr(1), addr(2), addr(3), 1, 2, 12, 0, 0,
                                         1e-6, None) == SHAPE
    assert lib.adaln_residual_gate_rmsnorm_scale_shift(
        addr(0), addr(1), None, None, addr(4), addr(5), addr(6), addr(7), 1, 2, 4096, 0, 0, 0,
        1e-6, None) == NULL
    assert lib.adaln_residual_gate_layernorm_modulate(
        addr(0), addr(1), addr(2), addr(4), addr(5), addr(6), addr(6), 1, 2, 3072, 0, 0, 0,
        1e-6, None) == OVERLAP
    assert lib.adaln_residual_gate_layernorm_modulate(
        None, None, None, None, None, None, None, 0, 2, 3072, 0, 0, 0, 1e-6, None) == OK
    assert lib.adaln_diag_round_bf16(None, None, -1, None) == SHAPE
    assert lib.adaln_diag_stream_copy(addr(0), addr(1), 24, None) == SHAPE
    assert lib.adaln_diag_stream_copy(addr(0), addr(1), -16, None) == SHAPE
    assert lib.adaln_diag_stream_copy(addr(0) + 8, addr(1), 32, None) == ALIGN
    assert lib.adaln_diag_stream_copy(None, addr(1), 32, None) == NULL
    assert lib.adaln_diag_stream_copy(addr(0), addr(0) + 16, 32, None) == OVERLAP
    assert lib.adaln_diag_stream_copy(None, None, 0, None) == OK
    for kind in (0, 1, 2):
        assert lib.adaln_diag_stream(kind, addr(0), addr(1), 24, 8, None) == SHAPE
        assert lib.adaln_diag_stream(kind, addr(0), addr(1), 32, 3, None) == VALUE
        assert lib.adaln_diag_stream(kind, addr(0), addr(1) + 8, 32, 8, None) == ALIGN
        assert lib.adaln_diag_stream(kind, addr(0), None, 32, 8, None) == NULL
        assert lib.adaln_diag_stream(kind, None, None, 0, 8, None) == OK
    assert lib.adaln_diag_stream(3, addr(0), addr(1), 32, 8, None) == VALUE
    assert lib.adaln_diag_stream(-1, addr(0), addr(1), 32, 8, None) == VALUE
    assert lib.adaln_diag_stream(0, None, addr(1), 32, 8, None) == NULL
    assert lib.adaln_diag_stream(1, None, addr(1), 32, 8, None) == NULL
    assert lib.adaln_diag_stream(1, addr(0) + 8, addr(1), 32, 8, None) == ALIGN
    # fill reads nothing: an unaligned src is not checked (the dst check still is)
    assert lib.adaln_diag_stream(2, addr(0) + 8, addr(1) + 8, 32, 8, None) == ALIGN
    assert lib.adaln_diag_stream(0, addr(0), addr(0) + 16, 64, 8, None) == OVERLAP
    # read writes only its folds (16 bytes per 4096*per bytes read) at the start of
    # dst: a dst starting inside src overlaps, one starting past the folds' reach of
    # src's end does not matter here (it would launch)
    assert lib.adaln_diag_stream(1, addr(0), addr(0) + 16, 4096 * 8, 8, None) == OVERLAP
    assert lib.adaln_diag_finalize(addr(0), addr(1), 4, 1, -1.0, None) == VALUE
    for H in (0, -1, 8193):
        assert lib.adaln_diag_finalize(addr(0), addr(1), 4, H, 1e-6, None) == SHAPE
    assert lib.adaln_diag_round_bf16(addr(0), addr(0) + 4, 8, None) == OVERLAP
    assert lib.adaln_diag_finalize(addr(0), addr(0) + 4, 8, 1, 1e-6, None) == OVERLAP
    assert lib.adaln_diag_quant_fp8(addr(0), addr(0) + 16, 8, addr(1), None) == OVERLAP


def test_binding_raises_adaln_error(lib):
    # a non-OK status from the library becomes AdalnError carrying the status
    with pytest.raises(A.AdalnError) as e:
        A.adaln_reduction_layout(12)
    assert e.value.status == SHAPE


def test_binding_rejects_host_tensors():
    """The Python binding passes device pointers only: host tensors are refused
    before the library is called."""
    import torch
    import diffusion_dit_adaln_amd as A
    x = torch.zeros((1, 4, 64), dtype=torch.bfloat16)
    v = torch.zeros((1, 64), dtype=torch.bfloat16)
    w = torch.zeros(64, dtype=torch.bfloat16)
    qs = torch.ones(1, dtype=torch.float32)
    calls = [
        lambda: A.adaln_layernorm_modulate(x, v, v),
        lambda: A.adaln_rmsnorm_scale_shift(x, w, v, v),
        lambda: A.adaln_residual_gate_rmsnorm_scale_shift(x, x, v, w, v, v),
        lambda: A.adaln_residual_gate_layernorm_modulate(x, x, v, v, v),
        lambda: A.adaln_layernorm_modulate_fp8_quant(x, v, v, qs),
        lambda: A.adaln_qk_rmsnorm_rope(torch.zeros((2, 3, 128), dtype=torch.bfloat16),
                                        torch.zeros((2, 3, 128), dtype=torch.bfloat16), None,
                                        None, torch.zeros((2, 128), dtype=torch.float32)),
        lambda: A.adaln_residual_gate_channel_first(torch.zeros((1, 8, 8), dtype=torch.bfloat16),
                                                    torch.zeros((1, 8, 8), dtype=torch.bfloat16),
                                                    torch.zeros((1, 8), dtype=torch.bfloat16)),
        lambda: A.adaln_diag_round_bf16(torch.zeros(8)),
        lambda: A.adaln_diag_finalize(torch.zeros(8)),
        lambda: A.adaln_diag_stream_copy(torch.zeros(8), torch.zeros(8)),
        lambda: A.adaln_diag_quant_fp8(torch.zeros(8), qs),
    ]
    for i, call in enumerate(calls):
        with pytest.raises(ValueError, match="CUDA"):
            call()
