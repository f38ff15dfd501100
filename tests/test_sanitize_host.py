"""The host-side C code of libdak (planner, turning points, host work-group
rule, argument validation and error state) built with AddressSanitizer and
UndefinedBehaviorSanitizer by g++ and driven on random and adversarial inputs
(tests/sanitize_planner_driver.cpp).  The driver also checks the turning
points against a scan of every h on tie-heavy ops and plans ops of up to 2^40
units.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tiered_memory_offloading_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_planner_and_validation_are_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "sanitize_planner")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-ffp-contract=off", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(ROOT, "tests", "sanitize_planner_driver.cpp"),
           os.path.join(CSRC, "planner.cpp"), os.path.join(CSRC, "errors.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    # verify_asan_link_order=0: the environment may preload a library of its
    # own ahead of the sanitizer runtime; that is not an error here.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "ok" in r.stdout
