"""Host-side sanitizer build: the library's workspace layout, argument checks and
key-split choice (csrc/host_layout.h, the same text the HIP library compiles)
built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and run
over many seeded problems, including the largest accepted sizes.  No GPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "log_domain_sinkhorn_half_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_logic_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", os.path.join(CSRC, "host_check.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert " 0 failures" in res.stdout, res.stdout
