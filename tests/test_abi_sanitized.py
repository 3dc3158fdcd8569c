"""The C ABI's argument validation under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only; no device is touched).

abi.cpp's host code is rebuilt with both sanitizers (UB aborts instead of recovering) and
linked, with the library's other objects as built, into tests/sanitize/abi_checks.cpp: a
driver that calls every entry point with arguments the checks must refuse (NULL and
misaligned pointers, short or overflowing leading dimensions, shapes past the size
limits, int64 extremes, unsupported schemes, roles and layouts, short workspaces) plus a
sweep of pql_kernel_name, and compares each status with the expected one.  Any heap /
stack overflow, signed overflow or other undefined behaviour on those paths fails the
test, as does a status mismatch."""
import os
import shutil
import subprocess
import tempfile

import pytest

from precision_quantized_linear_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _objects():
    objs = [os.path.join(B.OUT, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "abi.cpp"]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    return objs


@pytest.mark.skipif(not os.path.exists(B.hipcc()), reason="hipcc is not installed")
def test_abi_validation_under_asan_and_ubsan():
    objs = _objects()
    with tempfile.TemporaryDirectory() as tmp:
        flags = ["-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", B.CSRC,
                 "-Wno-unused-command-line-argument"]
        abi_o, drv_o, exe = (os.path.join(tmp, n) for n in ("abi_san.o", "drv.o", "abi_checks"))
        steps = [
            [B.hipcc(), *flags, f"--offload-arch={B.ARCH}", *SAN, "-x", "hip", "-c",
             os.path.join(B.CSRC, "abi.cpp"), "-o", abi_o],
            [B.hipcc(), *flags, *SAN, "-x", "c++", "-c", DRIVER, "-o", drv_o],
            [B.hipcc(), f"--offload-arch={B.ARCH}", *SAN, drv_o, abi_o, *objs, "-o", exe],
        ]
        for cmd in steps:
            r = subprocess.run(cmd, capture_output=True, text=True)
            assert r.returncode == 0, f"{' '.join(cmd[:3])} ...: {r.stderr[-2000:]}"
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        out = r.stdout + r.stderr
        assert r.returncode == 0 and "ok: 0 failures" in r.stdout, out[-4000:]
        assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
