"""The host contract of libh3.so under AddressSanitizer and
UndefinedBehaviorSanitizer, with the kernel-argument bounds checks compiled
in (ulysses_layout_amd/build_sanitized.py), on a machine without a GPU.

The checking build instruments the host code only.  The whole of
tests/test_host_contract.py runs against it in a child process that preloads
clang's ASan runtime: every rejection path, and every valid call up to its
launch (the full launch plan and its debug bounds checks, then H3_ERR_HIP
because there is no device).  Any sanitizer report or failed bounds check
ends the child with an error.
"""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SCRIPT = os.path.join(ROOT, "ulysses_layout_amd", "build_sanitized.py")


def _gpu_visible() -> bool:
    import torch
    return torch.cuda.device_count() > 0


pytestmark = pytest.mark.skipif(not os.path.exists(SCRIPT) or _gpu_visible(),
                                reason="host checking build: run where no GPU is visible")


def _builder():
    spec = importlib.util.spec_from_file_location("_h3_build_san", SCRIPT)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.timeout(600)
def test_host_contract_under_sanitizers():
    san = _builder()
    lib = san.build()
    dynsyms = subprocess.run(["nm", "-D", lib], stdout=subprocess.PIPE, text=True, check=True).stdout
    assert "__asan_report_load8" in dynsyms and "__ubsan_handle_" in dynsyms, "library is not instrumented"
    assert b"h3 debug bounds check failed" in open(lib, "rb").read(), "bounds checks not compiled in"
    env = dict(os.environ)
    env.update(LD_PRELOAD=san.asan_runtime(), H3_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_host_contract.py"),
                          "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                         stderr=subprocess.STDOUT, text=True, timeout=600)
    out = res.stdout
    assert "AddressSanitizer" not in out and "runtime error" not in out and "debug bounds" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out and "skipped" not in out.splitlines()[-1], out[-2000:]
