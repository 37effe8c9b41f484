"""The fused launch's plan (host logic, CPU): for every op, hidden size, row count,
batch split and set of resident counts, the row groups of one launch cover every row
exactly once; the grid and ring follow the documented rules; a group given to one
batch entry stays in it; a contiguous group's rows stay within 32-bit byte offsets.
The plan is the library's own host function (through the launch-plan diagnostic),
fed with resident counts like a device's: row groups with the default ring, the
one-slot ring and the two-row ring, and the CU count.  Launches of at least 2^25
elements (all ops but LN+FP8) take the one-shot grid: one pass of the default ring
per group, consecutive rows, as many groups as that takes."""
import numpy as np
import pytest

import diffusion_dit_adaln_amd as A

OPS = ["ln", "rms", "rg", "rgln", "lnq"]
INTERLEAVED = {"ln", "rgln", "lnq"}
# (deep, one-slot, two-row, CUs)
RESIDENT = [(1024, 1536, 1792, 256), (768, 0, 0, 256), (256, 512, 0, 64), (1, 1, 0, 1),
            (7, 0, 0, 7), (2560, 2560, 0, 256), (1024, 1536, 1280, 256), (1024, 1536, 1792, 0),
            (1024, 1536, 1280, 3)]
ONESHOT = 1 << 25  # elements per launch from which the one-shot grid is taken
# (rows, T): one batch entry, a few long ones, many short ones
SHAPES = [(1, 1), (3, 1), (7, 7), (7, 1), (100, 100), (100, 25), (4216, 4216), (4216, 527),
          (9216, 4608), (9216, 9216), (30001, 1579), (524287, 524287), (524288, 4096),
          (524288, 64), (8192, 8192), (64 * 15, 15)]


def default_slots(op, H):
    """The default ring depth of a layout: two for two-wave rows without the gate,
    else three up to 32 bf16 of activations per lane and two above."""
    w, _, c = A.adaln_reduction_layout(H)
    gated = op in ("rg", "rgln")
    if w == 2 and not gated:
        return 2
    return 3 if c * 8 * (2 if gated else 1) <= 32 else 2


def one_shot(op, rows, H):
    return op != "lnq" and rows * H >= ONESHOT


def rows_of(plan, rows):
    """Every row each group visits, as the kernel walks them, and the group of each."""
    g = np.arange(plan["groups"], dtype=np.int64)
    blk = g // plan["gpb"]
    blk_begin = blk * plan["blk_rows"]
    begin = blk_begin + (g - blk * plan["gpb"]) * plan["group_stride"]
    end = np.minimum(np.minimum(begin + plan["span"], rows), blk_begin + plan["blk_rows"])
    counts = np.maximum(0, (end - begin + plan["step"] - 1) // plan["step"])
    out = np.repeat(begin, counts)
    first = np.repeat(np.cumsum(counts) - counts, counts)
    out += (np.arange(out.size) - first) * plan["step"]
    return out, np.repeat(g, counts)


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("H", [8, 520, 1024, 2048, 3072, 4096, 4104, 6144, 8192])
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("res", RESIDENT)
def test_every_row_exactly_once(op, H, shape, res):
    rows, T = shape
    resident, resident_shallow, resident_two, cus = res
    plan = A.adaln_diag_launch_plan(op, rows, H, T, res[:3], cus)
    w, _, _ = A.adaln_reduction_layout(H)
    visited, group = rows_of(plan, rows)
    assert visited.size == rows
    assert np.array_equal(np.sort(visited), np.arange(rows))
    B = rows // T
    assert plan["block_threads"] == (256 if w == 1 else 64 * w)
    assert plan["blocks"] == ((plan["groups"] + 3) // 4 if w == 1 else plan["groups"])
    assert plan["blocks"] * plan["block_threads"] < 2**32
    if one_shot(op, rows, H):
        # one pass of the default ring per group, consecutive rows, any resident count
        S = default_slots(op, H)
        assert (plan["shallow"], plan["ring"], plan["slots"]) == (False, 0, S)
        assert (plan["span"], plan["group_stride"], plan["step"]) == (S, S, 1)
        assert plan["groups"] == plan["gpb"] == -(-rows // S) and plan["blk_rows"] == rows
        assert (plan["span"] + S) * 2 * H <= 2**31 - 1
    elif op in INTERLEAVED:
        shallow = resident_shallow > 0 and rows >= 3 * resident
        assert plan["shallow"] == shallow and plan["ring"] == (1 if shallow else 0)
        G = min(rows, resident_shallow if shallow else resident)
        per_entry = min(G // B, T) if B > 1 else 0
        assert plan["group_stride"] == 1 and plan["step"] == plan["gpb"]
        if per_entry > 0 and 16 * (G - per_entry * B) <= G:
            # each batch entry has its own groups, at most 1/16 of the slots idle
            assert (plan["gpb"], plan["blk_rows"], plan["span"]) == (per_entry, T, T)
            assert plan["groups"] == per_entry * B
            entries = np.zeros(plan["groups"], dtype=np.int64) - 1
            entries[group] = visited // T
            assert np.array_equal(entries[group], visited // T), "a group changes entry"
        else:
            assert plan["groups"] == plan["gpb"] == G
            assert plan["blk_rows"] == plan["span"] == rows
        if shallow:
            assert plan["slots"] == 1
    else:
        S = plan["slots"]
        # four-wave RMS rows take the one-slot ring for at most two rows per group
        shallow = (op == "rms" and w == 4 and resident_shallow > 0
                   and rows <= 2 * resident_shallow)
        assert plan["shallow"] == shallow and plan["step"] == 1
        if shallow:
            assert S == 1 and plan["ring"] == 1
        elif plan["ring"] == 2:
            # the two-row ring: ungated four-wave rows, only with its resident count
            assert op == "rms" and w == 4 and resident_two > 0 and cus > 0 and S == 2
        else:
            assert plan["ring"] == 0
        assert plan["gpb"] == plan["groups"] and plan["blk_rows"] == rows
        assert plan["span"] == plan["group_stride"] and plan["span"] % S == 0
        # the last pass reaches S rows past the span: still below 2^31 bytes
        assert (plan["span"] + S) * 2 * H <= 2**31 - 1
        # only the last group can be short
        assert plan["groups"] == -(-rows // plan["span"])


def test_two_row_ring_where_it_spreads_groups_more_evenly():
    # four-wave RMS rows at 8000 rows (just below the one-shot grid's 2^25 elements)
    # on a device like MI355X (resident counts of the weighted kernels: 4, 6 and 5
    # groups per CU): the two-row ring leaves the most loaded CU fewer rows
    res = (1024, 1536, 1280)
    for H in (4096, 4104):
        plan = A.adaln_diag_launch_plan("rms", 8000, H, 8000, res, 256)
        assert plan["ring"] == 2 and plan["slots"] == 2 and not plan["shallow"]
    # without its resident count or the CU count it is never chosen
    assert A.adaln_diag_launch_plan("rms", 8000, 4096, 8000, (1024, 1536, 0), 256)["ring"] == 0
    assert A.adaln_diag_launch_plan("rms", 8000, 4096, 8000, res, 0)["ring"] == 0
    # with one more two-row group per CU the three-row ring spreads 8000 rows better
    assert A.adaln_diag_launch_plan("rms", 8000, 4096, 8000, (1024, 1536, 1792), 256)["ring"] == 0
    # never for the gated op
    assert A.adaln_diag_launch_plan("rg", 8000, 4096, 8000, res, 256)["ring"] == 0


def test_large_launches_take_the_one_shot_grid():
    # from 2^25 elements per launch every op but LN+FP8 takes one pass of its default
    # ring per group, whatever fits on the device at once
    res = (1024, 1536, 1280)
    for op in ("ln", "rms", "rg", "rgln"):
        for rows, H in ((8192, 4096), (4096, 8192), (10923, 3072), (32768, 1024), (16384, 2048)):
            S = default_slots(op, H)
            plan = A.adaln_diag_launch_plan(op, rows, H, rows, res, 256)
            assert (plan["ring"], plan["slots"], plan["span"], plan["step"]) == (0, S, S, 1)
            assert plan["groups"] == -(-rows // S) > res[0]
            # two batch entries: the same ranges over the flat rows
            p2 = A.adaln_diag_launch_plan(op, 2 * rows, H, rows, res, 256)
            assert (p2["gpb"], p2["blk_rows"], p2["span"]) == (-(-2 * rows // S), 2 * rows, S)
        # one row fewer: the persistent grid (interleaved rows, or ranges of several
        # passes), a few groups per resident slot at most
        for rows, H in ((8191, 4096), (10922, 3072)):
            plan = A.adaln_diag_launch_plan(op, rows, H, rows, res, 256)
            S = default_slots(op, H)
            assert plan["groups"] <= 3 * 1536
            assert plan["step"] > 1 or plan["span"] > S
    # LN+FP8, bound by its arithmetic, keeps the persistent grid at any size
    plan = A.adaln_diag_launch_plan("lnq", 65536, 3072, 65536, res, 256)
    assert plan["groups"] <= 1536 and plan["ring"] == 1


def test_one_shot_grid_stays_below_2_32_work_items():
    # so many rows that one pass per group would pass 2^32 work-items: each group
    # takes whole passes more, and its rows stay within 32-bit byte offsets
    for op, rows, H in (("rms", 3 * 10**8, 8192), ("ln", 2**33, 8), ("rg", 2**31, 1024),
                        ("rgln", 5 * 10**8, 3072)):
        plan = A.adaln_diag_launch_plan(op, rows, H, rows, (1024, 0, 0), 256)
        S = plan["slots"]
        assert S == default_slots(op, H) and plan["span"] % S == 0 and plan["span"] > S
        assert plan["blocks"] * plan["block_threads"] <= 2**32 - 1
        assert plan["groups"] * plan["span"] >= rows > (plan["groups"] - 1) * plan["span"]
        assert (plan["span"] + S) * 2 * H <= 2**31 - 1
        # one pass fewer per group would not fit
        per = plan["span"] - S
        w, _, _ = A.adaln_reduction_layout(H)
        groups = -(-rows // per)
        blocks = -(-groups // 4) if w == 1 else groups
        assert blocks * plan["block_threads"] > 2**32 - 1


def test_persistent_grid_stays_below_2_32_work_items():
    # LN+FP8 keeps the persistent grid at any size: even with resident counts no
    # device has, its groups are capped so that the grid holds fewer than 2^32
    # work-items, and every row is still covered
    big = 2**31 - 1
    for rows, H in ((2**26, 3072), (2**28, 1024), (2**25, 8192)):
        plan = A.adaln_diag_launch_plan("lnq", rows, H, rows, (big, big, 0), 256)
        assert plan["blocks"] * plan["block_threads"] <= 2**32 - 1
        assert plan["step"] == plan["gpb"] == plan["groups"]
        assert plan["groups"] * -(-rows // plan["groups"]) >= rows


def test_interleaved_batch_entries_get_their_own_groups():
    # the FLUX.1 LayerNorm site [2, 4608, 3072] on 2560 resident groups: 1280 per entry
    plan = A.adaln_diag_launch_plan("lnq", 9216, 3072, 4608, (2560, 2560), 256)
    assert (plan["groups"], plan["gpb"], plan["blk_rows"], plan["step"]) == (2560, 1280, 4608, 1280)
    # 2560 groups over 7 entries would leave 5 slots idle (< 1/16): split
    assert A.adaln_diag_launch_plan("ln", 7 * 1024, 3072, 1024, (2560, 2560))["gpb"] == 365
    # 2560 groups over 1000 entries would idle 560 slots: one interleave over all rows
    plan = A.adaln_diag_launch_plan("ln", 1000 * 8, 3072, 8, (2560, 2560))
    assert (plan["groups"], plan["gpb"], plan["blk_rows"]) == (2560, 2560, 8000)


def test_plan_rejects_bad_arguments():
    with pytest.raises(ValueError):  # three resident counts at most
        A.adaln_diag_launch_plan("ln", 10, 1024, 10, (1024, 0, 0, 0))
    bad = [("ln", 0, 1024, 1, (1024, 0, 0), 0), ("ln", 10, 12, 10, (1024, 0, 0), 0),
           ("ln", 10, 1024, 10, (0, 0, 0), 0), ("ln", 10, 1024, 10, (2**31, 0, 0), 0),
           ("ln", 10, 1024, 10, (1024, 2**31, 0), 0), ("ln", 10, 1024, 10, (1024, 0, -1), 0),
           ("ln", 10, 1024, 10, (1024, 0, 2**31), 0), ("ln", 10, 1024, 10, (1024, 0, 0), -1),
           ("ln", 10, 1024, 10, (1024, 0, 0), 2**31)]
    for op, rows, H, T, res, cus in bad:
        with pytest.raises(A.AdalnError):
            A.adaln_diag_launch_plan(op, rows, H, T, res, cus)
    for T in (0, 3, 11, -1):  # T must divide rows
        with pytest.raises(A.AdalnError):
            A.adaln_diag_launch_plan("ln", 10, 1024, T, (1024, 0, 0))
