"""Host-side checks of bench.py (no GPU): the one-GPU rule and the link
between the committed profile summary and the kernel source it was taken on."""

import hashlib
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


def test_profile_traffic_is_tied_to_the_assembly_source():
    text = open(bench.PROFILE).read()
    recorded = [ln.split(": ")[1] for ln in text.splitlines() if "assembly.hip sha256" in ln]
    assert len(recorded) == 1
    now = hashlib.sha256(open(bench.ASSEMBLY_SRC, "rb").read()).hexdigest()
    got = bench.measured_traffic("L4096_N1700416_d2048", "auto")
    if recorded[0] == now:
        # the counters were taken on this source: the bytes are reported, and
        # they exceed the algorithmic bytes (every task reads a V row)
        assert isinstance(got, int) and got > 3.7e9
    else:
        assert got is None
    assert bench.measured_traffic("L4096_N280900_d768", "auto") is None


@pytest.mark.parametrize("name", ["L4096_N1700416_d2048"])
def test_profile_summary_names_its_command(name):
    text = open(bench.PROFILE).read()
    assert "rocprofv3" in text and "bench.py" in text and name in os.path.basename(bench.PROFILE)
