"""The host translation units of the library under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

prepare_host.cpp (sketch statistics with exact accumulators, device-layout
packing, the Householder / bisection / inverse-iteration eigen-solver of the
rank-r map, the host thread pool) and fault.cpp (the allocation fault injector)
are compiled with g++ and both sanitizers, together with the driver
tests/host/prepare_check.cpp, which prepares experts of several shapes and edge
rows on four threads and exercises the injector. Any sanitizer finding aborts
the program; any failed invariant makes it exit non-zero.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "activation_sparse_expert_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_preparation_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "prepare_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-ffp-contract=off", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "prepare_host.cpp"), os.path.join(CSRC, "fault.cpp"),
           os.path.join(ROOT, "tests", "host", "prepare_check.cpp"), "-o", exe, "-pthread"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.startswith("ok"), run.stdout
