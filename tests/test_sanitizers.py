"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU).

* The oracle (oracle/ds4o.c) is built with gcc and the sanitizers and driven over every
  function on small and edge-case inputs (tests/sanitize/oracle_driver.c).
* libds4attn's host side (argument validation, plans, workspace sizes) is built with the
  sanitizers on the host pass only (device code is built as usual and never runs here) and
  driven over every refusal rule and a sweep of size queries up to the documented limits
  (tests/sanitize/host_driver.cpp).
Either driver aborts on the first sanitizer report; both print "ok" when every call ended
with its documented result.
"""
import os
import shutil
import subprocess

import pytest

from sparse_compressed_kv_amd.build import SOURCES as LIB_SOURCES

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
# host pass only: each sanitizer flag follows -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{cmd[0]} failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_oracle_under_asan_ubsan():
    if not shutil.which("gcc"):
        pytest.skip("gcc not found")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-ffp-contract=off", "-Wall", "-Wextra", "-o", exe,
          os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "ds4o.c"), "-lm", "-lpthread"])
    r = _run([exe], env=ENV, timeout=300)
    assert r.stdout.strip().endswith("ok"), r.stdout


def test_library_host_side_under_asan_ubsan():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    os.makedirs(OUT, exist_ok=True)
    csrc = os.path.join(ROOT, "sparse_compressed_kv_amd", "csrc")
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
              "-I", os.path.join(ROOT, "include")]
    srcs = [(os.path.join(csrc, f), os.path.join(OUT, os.path.splitext(f)[0] + ".o")) for f in LIB_SOURCES]
    srcs.append((os.path.join(SAN, "host_driver.cpp"), os.path.join(OUT, "host_driver.o")))
    procs = [subprocess.Popen([HIPCC, *common, "-c", s, "-o", o], stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                              text=True) for s, o in srcs]
    for p, (s, _) in zip(procs, srcs):
        out, err = p.communicate()
        assert p.returncode == 0, f"{s}:\n{err[-3000:]}"
    exe = os.path.join(OUT, "host_driver")
    _run([HIPCC, "--offload-arch=gfx950", *HOST_SAN, "-o", exe, *[o for _, o in srcs]])
    r = _run([exe], env=ENV, timeout=300)
    assert r.stdout.strip().startswith("ok"), r.stdout
