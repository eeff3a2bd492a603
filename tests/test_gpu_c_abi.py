"""The relayouts driven from a plain C program (tests/c_gpu_relayout.c):
device memory from the HIP runtime, calls through include/h3.h, no Python or
torch in between.  Checks seq2head of every ragged rank (with and without a
chunk cap) and head2seq element by element against the partition's
closed-form mapping, and a misaligned pointer's rejection."""
import os
import shutil
import subprocess

import pytest

from tests.gpu_util import say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "ulysses_layout_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_relayouts_from_c(tmp_path):
    exe = str(tmp_path / "c_gpu_relayout")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_gpu_relayout.c"), "-o", exe, "-L", LIB_DIR, "-lh3",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{LIB_DIR}"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    say("relayouts from C: N=777, H=56, P=6, 3 planes")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(run.stdout)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "c gpu relayout: ok" in run.stdout
