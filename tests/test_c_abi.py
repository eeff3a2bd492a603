"""include/h3.h as plain C: tests/c_abi_check.c is compiled with gcc -std=c99
(warnings as errors), linked against the built libh3.so and run.  It calls the
host-only helpers and argument checks that return before any device work, so
it needs no GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "ulysses_layout_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_header_compiles_as_c_and_links(tmp_path):
    if not os.path.exists(os.path.join(LIB_DIR, "libh3.so")):
        pytest.fail("libh3.so is not built: run `python ulysses_layout_amd/build.py`")
    exe = str(tmp_path / "c_abi_check")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_check.c"), "-o", exe, "-L", LIB_DIR, "-lh3",
           f"-Wl,-rpath,{LIB_DIR}"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "c abi: ok" in run.stdout
