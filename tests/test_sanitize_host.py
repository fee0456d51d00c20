"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers, each built here and run as a subprocess:
* tests/sanitize/oracle_driver.c with oracle/pa_oracle.c (gcc, both sanitizers):
  every oracle entry point on small inputs with the edge cases the tests use;
* tests/sanitize/abi_driver.cpp with the library's sources (hipcc; the
  sanitizers instrument the host pass only, device code is built as usual):
  every entry point's argument validation, none of which reaches a launch.
A sanitizer report makes the driver exit non-zero; both must print "ok".
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-2000:] + r.stderr[-4000:]


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_san")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off", "-o", exe,
                           os.path.join(ROOT, "oracle", "pa_oracle.c"), os.path.join(SAN, "oracle_driver.c"), "-lm"])
    _run(exe)


def test_library_validation_under_host_asan_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from fp8_paged_kv_amd import build
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include")]
    procs, objs = [], []
    for src in build.SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([hipcc] + flags + build.EXTRA.get(src, []) +
                                      ["-c", os.path.join(build.CSRC, src), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    drv = str(tmp_path / "abi_driver.o")
    procs.append(subprocess.Popen([hipcc] + flags + ["-x", "c++", "-c", os.path.join(SAN, "abi_driver.cpp"), "-o", drv],
                                  stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p in procs:
        out, err = p.communicate(timeout=600)
        assert p.returncode == 0, err[-3000:]
    exe = str(tmp_path / "abi_san")
    subprocess.check_call([hipcc, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                           "-fsanitize=undefined", "-o", exe] + objs + [drv])
    _run(exe)
