"""The host-side index builder and validator under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): tests/host/index_harness.cpp builds and
validates indexes of every pattern kind into exactly sized buffers, corrupts
them, and checks the validator's verdicts."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_index_builder_under_sanitizers(tmp_path):
    exe = tmp_path / "index_harness"
    src = [os.path.join(ROOT, "tests", "host", "index_harness.cpp"),
           os.path.join(ROOT, "long_context_sparse_static_amd", "csrc", "block_index.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", *src, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    # verify_asan_link_order=0: the environment may preload another library
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "harness ok" in r.stdout, r.stdout + r.stderr
