"""The fused LayerNorm kernels compute rstd = RN(1/RN(sqrt(RN(RN(S/H) + eps)))) with
shorter exact steps when a wave's statistics are in range (a divide by H through the
rounded reciprocal with one exact correction, the hardware root and reciprocal with
exact residual fix-ups).  These host tests run those steps, in binary32 with fused
multiply-adds as on the device, over every case that the scaling argument leaves:
every significand of S for every H the library accepts, every v in [1, 4) for the
root, every significand for the reciprocal.  The device's own results are checked
over every non-negative statistic by the GPU finalize tests."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path_factory.mktemp("rstd") / "rstd_steps_check")
    subprocess.run([cc, "-O2", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "rstd_steps_check.c"), "-lm"], check=True)
    return exe


def run(exe, *args):
    out = subprocess.run([exe, *map(str, args)], check=True, capture_output=True,
                         text=True).stdout.split()
    assert out[0] == args[0] and out[1] == "failures"
    return int(out[2])


def over_all_h(exe, mode):
    """H = 8, 16, ..., 8192 split over worker processes."""
    bounds = [(8 + 1024 * i, 8 + 1024 * i + 1016) for i in range(8)]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        return sum(pool.map(lambda b: run(exe, mode, *b), bounds))


def test_divide_by_h_every_h_every_significand(checker):
    assert over_all_h(checker, "div") == 0


def test_uncorrected_divide_is_caught(checker):
    # the control: without the correction step a third of the quotients are off
    assert run(checker, "div0", 3072, 3072) > 1_000_000
    assert run(checker, "div0", 4096, 4096) == 0  # a power of two: exact either way


def test_root_fixup_every_v(checker):
    assert run(checker, "sqrt") == 0


def test_reciprocal_step_every_significand(checker):
    assert run(checker, "rcp") == 0
    # the one significand it misses; the kernels take the general divide there
    assert run(checker, "rcp_ones") > 0
