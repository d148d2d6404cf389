"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Two CPU-only builds: the float64 oracle (oracle/ct_oracle.c) with a driver
that runs every oracle entry point on small geometries of all four beams, and
the HIP library's host geometry code (frame validation, ray tables, the
adjoint's range bound: csrc/ct_geometry.cpp, no HIP) with a driver that runs
valid descriptors and the validation error paths.  Sanitizer reports abort
the drivers (no recovery), so a clean exit means no report.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, exe):
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", *SAN, "-pthread", "-I", os.path.join(ROOT, "oracle"),
          os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "ct_oracle.c"), "-lm", "-o", exe],
         exe)


def test_host_geometry_under_sanitizers(tmp_path):
    exe = str(tmp_path / "geometry_san")
    csrc = os.path.join(ROOT, "ray_driven_projector_amd", "csrc")
    _run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-I", csrc,
          os.path.join(HERE, "geometry_driver.cpp"), os.path.join(csrc, "ct_geometry.cpp"), "-o", exe], exe)
