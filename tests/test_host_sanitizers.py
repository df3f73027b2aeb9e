"""The host-CPU projection's C++ under AddressSanitizer + UndefinedBehaviorSanitizer and
under ThreadSanitizer (the worker pool's spin-then-sleep hand-off): a driver built from the
library's host source with g++ runs random layers on every instruction set the CPU has and
several thread counts. Needs g++ only, no GPU and no built library."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

SRC = [os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"),
       os.path.join(ROOT, "nvfp4_quantized_moe_02_amd", "csrc", "host_decode.cpp")]


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
@pytest.mark.parametrize("flags", [["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
                                   ["-fsanitize=thread"]], ids=["asan_ubsan", "tsan"])
def test_host_projection_under_sanitizer(flags, tmp_path):
    exe = str(tmp_path / "driver")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-pthread", "-fno-omit-frame-pointer", *flags, *SRC, "-o", exe],
                   check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1",
               ASAN_OPTIONS="halt_on_error=1:verify_asan_link_order=0")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "ok (0 failures)" in r.stdout
