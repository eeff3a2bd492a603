"""Debug build of libh3.so for host-side checking on a machine without a GPU.

Usage: ``python ulysses_layout_amd/build_sanitized.py``.  Every source is
compiled as in build.py plus ``-DH3_DEBUG_BOUNDS`` (bounds checks on every
kernel-argument table before its launch) and AddressSanitizer and
UndefinedBehaviorSanitizer on the HOST code only (each sanitizer flag is
scoped with -Xarch_host; the gfx950 device code is built exactly as in the
release library).  The result is ``ulysses_layout_amd/_build_san/libh3_san.so``;
load it through the binding with ``H3_LIBRARY=<that path>`` in a process that
preloads clang's ASan runtime (``asan_runtime()``).  It is a checking build:
nothing in the package or the tests loads it by default.
"""
from __future__ import annotations

import glob
import importlib.util
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
_spec = importlib.util.spec_from_file_location("_h3_build", os.path.join(PKG, "build.py"))
_build = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(_build)

OUT_DIR = os.path.join(PKG, "_build_san")
LIB = os.path.join(OUT_DIR, "libh3_san.so")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = [f for f in _build.HIP_FLAGS if f != "-O3"] + ["-O1", "-g", "-DH3_DEBUG_BOUNDS"] + SAN_HOST


def asan_runtime() -> str:
    """clang's shared ASan runtime (it also carries the UBSan handlers)."""
    res = subprocess.run([_build.hipcc(), "--print-resource-dir"], stdout=subprocess.PIPE, text=True)
    hits = glob.glob(os.path.join(res.stdout.strip(), "lib", "linux", "libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang's libclang_rt.asan-x86_64.so not found")
    return hits[0]


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_build.hipcc(), *FLAGS, "-c", os.path.join(_build.CSRC, src), "-o", obj]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}")
    return obj


def build() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(_build.SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, _build.SOURCES))
    cmd = [_build.hipcc(), "-shared", "-fPIC", f"--offload-arch={_build.ARCH}", "-shared-libasan", *SAN_HOST,
           "-o", LIB, *objs]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError("link of libh3_san.so failed:\n" + res.stdout)
    return LIB


if __name__ == "__main__":
    print("built", build(), "; preload", asan_runtime())
    sys.exit(0)
