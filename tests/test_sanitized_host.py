"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The library's host code (argument validation, workspace layouts, launch
  planning in abi.cpp, step.cpp and the host side of the .hip files) is built
  with both sanitizers on the host compilation only (the device code is built
  as usual and never runs here), linked into tests/sanitize/abi_checks.cpp, and
  run: every call there is rejected on the host or is a size query, including
  40,000 randomized size queries.
* The CPU oracle (oracle/oracle.c) is built with gcc and both sanitizers into
  tests/sanitize/oracle_checks.c, which runs every oracle function on seeded
  ragged inputs and checks a property of each result.

Either program fails on an unexpected return code or a failed check, and the
sanitizers abort it on any memory error or undefined behaviour.
"""
import concurrent.futures
import os
import shutil
import subprocess
import tempfile

import pytest

from sequence_decode_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
# host compilation only: each -fsanitize= goes after -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.fixture(scope="module")
def tmp():
    d = tempfile.mkdtemp(prefix="sd_sanitize_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_abi_host_code_under_sanitizers(tmp):
    hipcc = B.hipcc()
    flags = [f for f in B.HIPFLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_SAN

    def compile_one(src):
        obj = os.path.join(tmp, src + ".o")
        _run([hipcc, *flags, *B.EXTRA.get(src, []), "-c", os.path.join(B.CSRC, src), "-o", obj])
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=6) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    drv = os.path.join(tmp, "abi_checks.o")
    _run([hipcc, *flags, "-c", os.path.join(SAN, "abi_checks.cpp"), "-o", drv])
    exe = os.path.join(tmp, "abi_checks")
    _run([hipcc, "--offload-arch=gfx950", *HOST_SAN, *objs, drv, "-o", exe])
    r = _run([exe], env=ENV, timeout=120)
    assert "abi checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_oracle_under_sanitizers(tmp):
    exe = os.path.join(tmp, "oracle_checks")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-Wall",
          "-Wno-unknown-pragmas", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer", os.path.join(SAN, "oracle_checks.c"),
          os.path.join(ROOT, "oracle", "oracle.c"), "-o", exe, "-lm"])
    r = _run([exe], env=ENV, timeout=120)
    assert "oracle checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
