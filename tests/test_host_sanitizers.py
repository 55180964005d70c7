"""The host-side code under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): the launcher's planning (launcher.cpp, which has no HIP dependency)
over a grid of shapes, forced configurations and device sizes including the
extremes of the argument ranges, and the CPU oracle on small and degenerate
products, built with g++/gcc and run by tests/hostsan/host_driver.cpp.  Any
sanitizer report fails the run."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs the host gcc/g++")
def test_host_code_under_sanitizers():
    with tempfile.TemporaryDirectory() as tmp:
        obj = os.path.join(tmp, "oracle.o")
        exe = os.path.join(tmp, "host_driver")
        subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-ffp-contract=off", *SAN,
                        "-c", os.path.join(ROOT, "oracle", "sdt_oracle.c"), "-o", obj],
                       check=True, capture_output=True, text=True)
        subprocess.run(["g++", "-std=c++17", "-O1", "-g", *SAN,
                        "-I", os.path.join(ROOT, "include"),
                        "-I", os.path.join(ROOT, "shape_driven_tile_amd", "csrc"),
                        os.path.join(ROOT, "tests", "hostsan", "host_driver.cpp"),
                        os.path.join(ROOT, "shape_driven_tile_amd", "csrc", "launcher.cpp"),
                        obj, "-fopenmp", "-lm", "-o", exe],
                       check=True, capture_output=True, text=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
        report = r.stdout + r.stderr
        assert r.returncode == 0, report
        assert "runtime error" not in report and "Sanitizer" not in report, report
        assert "shape plans" in r.stdout
