"""Host-side bounds checks of the fused forward's launch plan (no GPU).

tests/plan_check.cpp replays, with the offset helpers the kernel uses, every index the
fused kernel derives from the plan over a sweep of (n, D, n_alpha, T) and checks it
against the extent of the buffer it addresses; it is built here with g++.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_plan_indices_stay_in_bounds(tmp_path):
    exe = tmp_path / "plan_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall",
                    f"-I{os.path.join(ROOT, 'mhc_hyper_connection_amd', 'csrc')}",
                    os.path.join(HERE, "plan_check.cpp"), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok ")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_backward_plan_indices_stay_in_bounds(tmp_path):
    exe = tmp_path / "bwd_plan_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall",
                    f"-I{os.path.join(ROOT, 'mhc_hyper_connection_amd', 'csrc')}",
                    os.path.join(HERE, "bwd_plan_check.cpp"), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok ")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_single_read_wait_counts(tmp_path):
    # the counts the single-read kernel's compute waves wait their x loads down to, against
    # a replay of the memory operations they issue (tests/wait_count_check.cpp)
    exe = tmp_path / "wait_count_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall",
                    f"-I{os.path.join(ROOT, 'mhc_hyper_connection_amd', 'csrc')}",
                    os.path.join(HERE, "wait_count_check.cpp"), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok ")
