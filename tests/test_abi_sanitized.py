"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/abi_check.cpp calls every entry point with invalid arguments, N = 0 and the
largest sizes the ABI accepts (nothing is launched, no pointer is dereferenced).  It is
linked with eql_api.hip rebuilt with the sanitizers on its host code only (device
code is never instrumented) and with the library's other objects from the last full
build.  Runs on the CPU; a sanitizer report or a failed check fails the test.
"""
import os
import subprocess

import pytest

from group_circulant_linear_p4_amd import build as B

SAN = os.path.join(B.BUILD, "sanitize")
# Host-only instrumentation: each sanitizer flag goes to the host compilation and link.
SAN_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
             "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer").split()


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("%s\n%s\n%s" % (" ".join(cmd), res.stdout[-4000:], res.stderr[-8000:]))


def build_abi_check() -> str:
    others = [os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "eql_api.hip"]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        pytest.skip("library objects not built (run the full build first): %s" % ", ".join(missing))
    os.makedirs(SAN, exist_ok=True)
    api = os.path.join(SAN, "eql_api.o")
    drv = os.path.join(SAN, "abi_check.o")
    exe = os.path.join(SAN, "abi_check")
    flags = [f for f in B.CFLAGS if f != "-O3"] + ["-O1"] + SAN_FLAGS
    _run([B.hipcc(), *flags, "-c", os.path.join(B.CSRC, "eql_api.hip"), "-o", api])
    _run([B.hipcc(), *flags, "-x", "hip", "-c", os.path.join(os.path.dirname(__file__), "abi_check.cpp"), "-o", drv])
    _run([B.hipcc(), "--offload-arch=" + B.ARCH, *SAN_FLAGS, api, drv, *others, "-o", exe])
    return exe


def test_abi_host_code_under_asan_and_ubsan():
    exe = build_abi_check()
    env = dict(os.environ)
    # The HIP runtime's own allocations at exit are not this library's: leaks are not
    # checked; any other report aborts.
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-6000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert "0 failed" in res.stdout, out[-6000:]
