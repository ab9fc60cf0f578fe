"""Host-side checks of bench.py (no GPU): the one-GPU rule and the link
between the committed profile summary and the kernel source it was taken on."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


PROFILED = ["L4096_N1700416_d2048", "L4096_N1048576_d1024", "L4096_N280900_d768"]


@pytest.mark.parametrize("name", PROFILED)
def test_profile_traffic_is_tied_to_the_kernel_sources(name):
    text = open(bench.profile_path(name)).read()
    recorded = [ln.rsplit(": ", 1)[1] for ln in text.splitlines()
                if ln.lstrip("- ").startswith("kernel sources sha256")]
    assert len(recorded) == 1
    got = bench.measured_traffic(name, "auto")
    if recorded[0] == bench.sources_sha256():
        # the counters were taken on these sources: the bytes are reported
        assert isinstance(got, int) and got > 0
    else:
        assert got is None
    assert bench.measured_traffic(name, "no_such_assembly") is None


def test_workload_without_a_profile_has_no_traffic():
    assert bench.measured_traffic("tiny_L64_N1024_d64_f32", "auto") is None


@pytest.mark.parametrize("name", PROFILED)
def test_profile_summary_names_its_command(name):
    path = bench.profile_path(name)
    text = open(path).read()
    assert "rocprofv3" in text and "bench.py" in text and f"--workload {name}" in text
