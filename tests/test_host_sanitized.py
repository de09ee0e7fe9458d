"""The library's host code (trie, layout, validation, placement, row planner, GDN chain plan) built with
AddressSanitizer and UndefinedBehaviorSanitizer and driven through its C entry points on random forests,
workload-sized rows and malformed inputs (tests/sanitize/host_driver.cpp).  CPU only: the host C++ is
compiled with g++, no device code is involved."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "host_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"),
           os.path.join(ROOT, "prefix_tree_packed_dfs_amd", "csrc", "host.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"build failed:\n{r.stderr[-4000:]}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, f"sanitized run failed ({r.returncode}):\n{r.stdout[-2000:]}\n{r.stderr[-6000:]}"
    assert "all checks passed" in r.stdout
