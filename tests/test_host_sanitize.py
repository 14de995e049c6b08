"""The host-only entry points (row plan, score blocks, score width, window
size) built with a host compiler under the address and undefined-behaviour
sanitizers and driven over random and boundary inputs by
tests/host_plan_check.cpp. CPU only."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_host_plan_under_sanitizers(tmp_path):
    exe = tmp_path / "host_plan_check"
    cmd = ["g++", "-x", "c++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "sparse_attention_decode_02_amd", "csrc", "host_plan.hip"),
           os.path.join(HERE, "host_plan_check.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    # verify_asan_link_order=0: the environment may preload a library ahead
    # of the sanitizer runtime; that is tolerated, not changed.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe), "1500"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
