"""The native block manager under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only, built with g++): tests/bm_stress.cpp drives random operation
sequences through the C ABI and checks the state after each one."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "paged_kv_cache_75_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_block_manager_under_sanitizers(tmp_path):
    exe = str(tmp_path / "bm_stress")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(HERE, "bm_stress.cpp"), os.path.join(CSRC, "pa_block_manager.cpp"),
           os.path.join(CSRC, "pa_sha256.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    # verify_asan_link_order=0: the runtime need not be first among preloaded
    # libraries of the environment the test runs in
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "copy-on-write pairs" in r.stdout
