"""The kernels' workgroup -> tile schedules, checked on the host.

tests/schedule_check.hip includes the same fa_schedule.hpp the kernels use,
walks every workgroup index of ~50k grid shapes (dense and packed forward,
split-key forward, both backward passes, decoding) and requires each tile to
be issued exactly once; under causal masking also that pairs join tile t with
tile n-1-t, that the split tail runs heaviest first on each XCD, and that a
dense grid has no empty workgroup.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_44_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not shutil.which(HIPCC), reason="hipcc not found")
def test_every_tile_issued_exactly_once(tmp_path):
    exe = str(tmp_path / "schedule_check")
    build = subprocess.run([HIPCC, "-std=c++17", "-O1", "--offload-host-only", "-x", "hip",
                            "-I" + CSRC, os.path.join(ROOT, "tests", "schedule_check.hip"),
                            "-o", exe], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.startswith("ok"), run.stdout + run.stderr
    assert int(run.stdout.split()[1]) > 50000
