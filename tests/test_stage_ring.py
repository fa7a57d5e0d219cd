"""The pinned ring that carries parameter tables to the device
(`csrc/stage_ring.h`), checked on the host: a simulated stream runs the
enqueued copies in order a few at a time while tables keep arriving, and no
region may be written again before the copy from it has run. The same
simulation run with bookkeeping that checks only the oldest listed use (a
region skipped at the ring's end then hides later ones) or nothing at all must
catch the overwrite, so the check itself is shown to bite."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "lora_swiglu_mlp_amd", "csrc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no g++")
    exe = str(tmp_path_factory.mktemp("ring") / "stage_ring_check")
    subprocess.run([cxx, "-std=c++17", "-O2", "-Wall", "-Werror", "-I", CSRC,
                    os.path.join(HERE, "stage_ring_check.cpp"), "-o", exe], check=True)
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_ring_never_writes_a_region_before_its_copy_ran(checker, seed):
    r = subprocess.run([checker, "ring", str(seed), "200000"], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    staged, fallback = (int(v) for v in r.stdout.split()[2::2])
    assert staged > 150000 and fallback > 0  # both paths taken


@pytest.mark.parametrize("mode", ["frontonly", "nocheck"])
def test_weaker_bookkeeping_is_caught(checker, mode):
    r = subprocess.run([checker, mode, "1", "200000"], capture_output=True, text=True)
    assert r.returncode == 3, r.stdout + r.stderr
    assert "written over" in r.stdout
