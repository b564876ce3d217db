"""Host AddressSanitizer + UndefinedBehaviorSanitizer runs (CPU only):

* the fp64 oracle (oracle/lisa_oracle.c) under a driver that reaches its edge
  cases (tests/sanitize/oracle_driver.c), built with gcc;
* the C ABI's validation layer: the library's sources built with hipcc, the
  host code instrumented and the device code not, under a driver that makes
  every call that must return before any HIP call (tests/sanitize/
  abi_driver.cpp).

A sanitizer report aborts the driver, so both must exit 0 and print "ok".
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (cmd, r.stdout[-3000:], r.stderr[-3000:])
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-fopenmp", *SAN, os.path.join(HERE, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "lisa_oracle.c"), "-o", exe, "-lm"])
    r = _run([exe], env=ENV, timeout=300)
    assert r.stdout.strip().endswith("ok"), r.stdout


HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_validation_under_asan_ubsan(tmp_path):
    from hybrid_linear_top_amd import build as hb
    # host code instrumented, device code not: each -fsanitize= goes to the host pass only
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f] if f.startswith("-fsanitize") or f.startswith("-fno-sanitize") else [f]
    objs = []
    import concurrent.futures as cf

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        _run([HIPCC, *hb.FLAGS, *host_san, "-O1", "-c", os.path.join(hb.CSRC, src), "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, hb.SOURCES))
    drv = str(tmp_path / "abi_driver.o")
    _run([HIPCC, "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"), *host_san, "-O1", "-c",
          os.path.join(HERE, "abi_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_driver")
    _run([HIPCC, f"--offload-arch={hb.ARCH}", *host_san, drv, *objs, "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert r.stdout.strip().endswith("ok"), r.stdout
