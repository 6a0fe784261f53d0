"""The host half of libpkv (host.cpp) under AddressSanitizer and UBSan.

host.cpp is compiled with g++ on the CPU together with host_fuzz.cpp, a
driver that runs random (valid and invalid) operation sequences through the
C ABI: allocator, copy-on-write, retention pool, prepare_step, planner and
table validation.  Any out-of-bounds access, use after free, leak or
undefined behaviour aborts the driver.  No GPU code is built or run.
"""

import os
import shutil
import subprocess

import pytest

from conftest import ROOT

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")


def test_host_library_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "host_fuzz"
    flags = ["-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
             "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include")]
    srcs = [os.path.join(ROOT, "tests", "host_fuzz.cpp"),
            os.path.join(ROOT, "pagedattention_pkv_store_amd", "csrc", "host.cpp")]
    subprocess.run(["g++", *flags, *srcs, "-o", str(exe)], check=True, capture_output=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "fuzz done" in r.stdout
