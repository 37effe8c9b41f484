"""The fused kernel's launch plan (host logic, CPU): for every op, hidden size and
row count, the row groups of one launch cover every row exactly once, the grid and
ring settings follow the documented rules, and a contiguous group's rows stay within
32-bit byte offsets.  The plan is the library's own host function (through the
launch-plan diagnostic), fed with resident counts like the device's."""
import numpy as np
import pytest

import diffusion_dit_adaln_amd as A

OPS = ["ln", "rms", "rg", "rgln", "lnq"]
INTERLEAVED = {"ln", "rgln", "lnq"}
RESIDENT = [(1024, 1536), (768, 0), (256, 512), (1, 1), (7, 0)]


def rows_of(plan, rows):
    """Every row each group visits, as the kernel walks them."""
    g = np.arange(plan["groups"], dtype=np.int64)
    begin = g * plan["group_stride"]
    end = np.minimum(begin + plan["span"], rows)
    counts = np.maximum(0, (end - begin + plan["step"] - 1) // plan["step"])
    out = np.repeat(begin, counts)
    first = np.repeat(np.cumsum(counts) - counts, counts)
    out += (np.arange(out.size) - first) * plan["step"]
    return out


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("H", [8, 520, 1024, 2048, 3072, 4096, 4104, 8192])
@pytest.mark.parametrize("rows", [1, 3, 7, 100, 4216, 9216, 30001, 524287])
@pytest.mark.parametrize("res", RESIDENT)
def test_every_row_exactly_once(op, H, rows, res):
    resident, resident_shallow = res
    plan = A.adaln_diag_launch_plan(op, rows, H, resident, resident_shallow)
    w, _, _ = A.adaln_reduction_layout(H)
    visited = rows_of(plan, rows)
    assert visited.size == rows
    assert np.array_equal(np.sort(visited), np.arange(rows))
    assert plan["block_threads"] == (256 if w == 1 else 64 * w)
    assert plan["blocks"] == ((plan["groups"] + 3) // 4 if w == 1 else plan["groups"])
    if op in INTERLEAVED:
        shallow = resident_shallow > 0 and rows >= 3 * resident
        assert plan["shallow"] == shallow
        assert plan["groups"] == min(rows, resident_shallow if shallow else resident)
        assert plan["group_stride"] == 1 and plan["step"] == plan["groups"]
        if shallow:
            assert plan["slots"] == 1
    else:
        S = plan["slots"]
        assert plan["shallow"] == 0 and plan["step"] == 1
        assert plan["span"] == plan["group_stride"] and plan["span"] % S == 0
        # the last pass reaches S rows past the span: still below 2^31 bytes
        assert (plan["span"] + S) * 2 * H <= 2**31 - 1
        # only the last group can be short
        assert plan["groups"] == -(-rows // plan["span"])


def test_contiguous_groups_capped_by_32_bit_offsets():
    # so many rows per group that the span would pass 2^31 bytes: the span is
    # capped and the group count grows instead
    rows, H = 3 * 10**8, 8192
    plan = A.adaln_diag_launch_plan("rms", rows, H, 1024, 0)
    S = plan["slots"]
    assert (plan["span"] + S) * 2 * H <= 2**31 - 1
    assert plan["groups"] * plan["span"] >= rows > (plan["groups"] - 1) * plan["span"]


def test_plan_rejects_bad_arguments():
    with pytest.raises(A.AdalnError):
        A.adaln_diag_launch_plan("ln", 0, 1024, 1024)
    with pytest.raises(A.AdalnError):
        A.adaln_diag_launch_plan("ln", 10, 12, 1024)
    with pytest.raises(A.AdalnError):
        A.adaln_diag_launch_plan("ln", 10, 1024, 0)
