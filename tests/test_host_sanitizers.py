"""The host-only parts of the library (config validation, sizes, read
accounting, the sketch pack with its worker threads) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer and driven through the C ABI
(tests/host_sanitize/pack_driver.cpp): no memory error, no undefined
behaviour, and non-finite weights are rejected."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "calibration_free_channel_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_pack_under_sanitizers(tmp_path):
    exe = str(tmp_path / "pack_driver")
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-pthread", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(ROOT, "tests", "host_sanitize", "pack_driver.cpp"),
           os.path.join(CSRC, "common.cpp"), os.path.join(CSRC, "pack_host.cpp"), "-o", exe]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert res.returncode == 0, res.stdout
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env,
                         timeout=600)
    assert run.returncode == 0, run.stdout
