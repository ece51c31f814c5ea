"""The library's host code under AddressSanitizer and UBSan (CPU only).

The library sources and the CPU walk of the kernel (tests/kernel_emu.cpp) are
built with host-side instrumentation (each sanitizer flag behind -Xarch_host, so
no GPU code is instrumented) and driven by tests/asan_driver.py in a child process
that preloads the sanitizer runtime: host preparation, the kernel's tile walk, the
copy-engine plan, the span-record arena and the validation error paths, all
compared with the oracle.  Any sanitizer report fails the test.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

from paged_layout_transfer_amd import _build

HERE = os.path.dirname(os.path.abspath(__file__))


def _runtime() -> str | None:
    found = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(_build.HIPCC)), "llvm", "lib", "clang",
                                          "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    found += sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[0] if found else None


@pytest.mark.timeout(900)
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    rt = _runtime()
    if rt is None:
        pytest.skip("no sanitizer runtime next to the compiler")
    out = str(tmp_path / "libemu_asan.so")
    flags = [f for f in _build.FLAGS if f != "-fvisibility=hidden"]
    cmd = [_build.HIPCC, *flags,
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-shared-libsan", "-I", os.path.join(_build.ROOT, "include"), "-I", _build.CSRC,
           *_build.SOURCES, os.path.join(HERE, "kernel_emu.cpp"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, os.path.join(HERE, "asan_driver.py"), out], env=env,
                       capture_output=True, text=True, timeout=800)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
