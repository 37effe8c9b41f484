"""Host-side logic of bench.py (CPU only): the one-GPU guard, workload sizes and
algorithmic bytes, the kernel-source hash that keys the committed counters, and the
counter summary being used only while that hash matches."""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name,op,rows,nbytes", [
    ("ln_1x128x2048", "ln", 128, 4 * 128 * 2048),
    ("rms_1x4216x4096", "rms", 4216, 4 * 4216 * 4096),
    ("rg_rms_2x1140x4096", "rg", 2280, 8 * 2280 * 4096),
    ("ln_2x4608x3072", "ln", 9216, 4 * 9216 * 3072),
    ("ln_1x4333x3072", "ln", 4333, 4 * 4333 * 3072),
    ("rg_ln_2x4096x3072", "rgln", 8192, 8 * 8192 * 3072),
    ("ln_fp8_2x4608x3072", "lnq", 9216, 3 * 9216 * 3072),
    ("qk_rmsnorm_rope_4608x24x128", "qk", 4608 * 48, 8 * 4608 * 24 * 128 + 4 * 4608 * 128),
    ("rg_channel_first_2x3072x4608", "cf", 9216, 6 * 2 * 3072 * 4608),
])
def test_workload_sizes(name, op, rows, nbytes):
    wl = bench.workload(name)
    assert wl.name == name and wl.op == op
    assert bench.workload_rows(wl) == rows
    assert wl.algorithmic_bytes() == nbytes
    assert bench.describe(wl)
    sha = bench.inputs_sha256(wl)
    assert sha and all(len(v) == 16 for v in sha.values())


def test_headline_config_is_the_largest_target_config():
    # the metric names no configuration: the timed line is the largest configuration
    # with the bandwidth target, the FLUX.1 LayerNorm site [2,4608,3072]
    assert bench.HEADLINE in bench.WORKLOAD_NAMES
    wl = bench.workload(bench.HEADLINE)
    assert wl.x.shape == (2, 4608, 3072) and wl.op == "ln"
    assert wl.algorithmic_bytes() == 113246208
    sizes = {n: bench.workload(n).algorithmic_bytes() for n in bench.TARGET_CONFIGS}
    assert max(sizes, key=sizes.get) == bench.HEADLINE
    assert set(bench.TARGET_CONFIGS) == {"rms_1x4216x4096", "rg_rms_2x1140x4096",
                                         "ln_2x4608x3072", "ln_1x4333x3072"}


def test_profile_tables_used_only_for_the_same_kernel_source(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_profile_table("t.txt", 0, 3) == {}
    f = tmp_path / "profiles" / "t.txt"
    f.write_text(f"# a comment\n# kernel_src_sha = {bench.kernel_src_sha()}\n"
                 "w1 | k | 10 | 15009.8 | x\nw2 | k | 10 | notanumber\n")
    assert bench.load_profile_table("t.txt", 0, 3) == {"w1": 15009.8}
    f.write_text("# kernel_src_sha = 0000000000000000\nw1 | k | 10 | 15009.8\n")
    assert bench.load_profile_table("t.txt", 0, 3) == {}


def test_inputs_are_seeded():
    a = bench.inputs_sha256(bench.workload("rg_rms_2x1140x4096"))
    b = bench.inputs_sha256(bench.workload("rg_rms_2x1140x4096"))
    assert a == b


def test_kernel_hash_ignores_comments_and_blank_space(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f(int a) {\n  return a + 1; // one\n}\n/* block\n comment */\n")
    monkeypatch.setattr(bench, "KERNEL_SRCS", [str(src)])
    h0 = bench.kernel_src_sha()
    src.write_text("int f(int a) {   return a + 1; // other words\n}\n\n\n")
    assert bench.kernel_src_sha() == h0
    src.write_text("int f(int a) { return a + 2; }\n")
    assert bench.kernel_src_sha() != h0


def test_counters_used_only_for_the_same_kernel_source(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_counters("w") is None                      # no summary
    f = tmp_path / "profiles" / "counters_w.txt"
    f.write_text(f"# note = ignored\nkernel_src_sha = {bench.kernel_src_sha()}\n"
                 "traffic_bytes_per_dispatch = 12345\n")
    assert bench.load_counters("w") == 12345.0
    f.write_text("kernel_src_sha = 0000000000000000\ntraffic_bytes_per_dispatch = 12345\n")
    assert bench.load_counters("w") is None                      # another source


def test_cpu_baseline_on_a_small_workload():
    wl = bench.workload("ln_1x128x2048")
    out = bench.cpu_baseline(wl, 0.05)
    assert out["kind"] == "oracle" and out["cores"] == 1 and out["value"] > 0
    assert out["unit"] == "GB/s" and "pinned to core" in out["sample"]
    if len(__import__("os").sched_getaffinity(0)) > 1:
        par = out["all_cores"]
        assert par["cores"] > 1 and par["equals_single_core"] is True and par["value"] > 0
    # the comparison with a GPU output of the same inputs (here the oracle's own bits)
    from oracle import oracle as O
    y = O.layernorm_modulate(wl.x, wl.scale, wl.shift, wl.eps)
    assert bench.cpu_baseline(wl, 0.01, y_gpu=[y])["gpu_output_equals_oracle"] is True
    y2 = y.copy()
    y2.flat[0] ^= 1
    assert bench.cpu_baseline(wl, 0.01, y_gpu=[y2])["gpu_output_equals_oracle"] is False
