"""Host-side logic of bench.py (no GPU): which runs an invocation times, where the roofline's
traffic figure comes from, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_default_runs_end_with_the_headline():
    runs = bench.select_runs(None, False)
    assert runs == list(bench.RUNS)
    assert runs[-1] == bench.HEADLINE == ("fp8_block_dit", "fp8_block128")


def test_all_puts_the_extra_runs_before_the_headline():
    runs = bench.select_runs(None, True)
    assert runs[-1] == bench.HEADLINE
    assert runs[:len(bench.RUNS) - 1] == list(bench.RUNS[:-1])
    assert runs[len(bench.RUNS) - 1:-1] == list(bench.EXTRA)
    assert ("load_and_dequant", "w4a16_asym+fp8_block128") in runs


@pytest.mark.parametrize("only,want", [
    ("fp8_block_dit", [("fp8_block_dit", "fp8_block128")]),           # a default name: its default run only
    ("fp8_row_dit", [("fp8_row_dit", "fp8_row")]),
    ("mx_video_dit:mxfp4", [("mx_video_dit", "mxfp4")]),
    ("fp8_row_dit:int8_row", [("fp8_row_dit", "int8_row")]),          # an --all entry by NAME:SCHEME
    ("load_and_dequant", [("load_and_dequant", "w4a16_asym+fp8_block128")]),   # a name only --all has
    ("no_such_workload", []),
])
def test_only_selects(only, want):
    assert bench.select_runs(only, False) == want


def test_traffic_comes_only_from_a_summary_of_the_current_kernel_source(tmp_path, monkeypatch):
    # the committed summaries carry the SHA of the source they were measured on
    assert bench.measured_traffic("k_gemm_block256__fp8_block_dit.md") == 1098938879
    assert isinstance(bench.measured_traffic("k_gemm32_mx__mx_video_dit.md", "traffic_bytes_per_launch_mxfp4"), int)
    assert bench.measured_traffic("no_such_profile.md") is None
    # a summary taken on another source gives no figure
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "stale.md").write_text("traffic_bytes_per_launch: 123\nkernel_source: bench.py\n"
                                   "kernel_source_sha256_16: 0000000000000000\n")
    (tmp_path / "bench.py").write_text("# not the source the figure was taken on\n")
    monkeypatch.setattr(bench.os.path, "abspath", lambda p: str(tmp_path / "bench.py"))
    assert bench.measured_traffic("stale.md") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
