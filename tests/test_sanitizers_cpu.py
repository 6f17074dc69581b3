"""Host sanitizer runs (CPU only): the fp64 oracle and the host side of
libtrimul built with AddressSanitizer and UndefinedBehaviorSanitizer (leak
detection on), each driven by a C program under tests/sanitize/ that must
exit 0 with no sanitizer report.  The library's device code is compiled
normally; only its host code is instrumented."""
import concurrent.futures as cf
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "OMP_NUM_THREADS": "2"}
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fopenmp", os.path.join(ROOT, "oracle", "trimul_oracle.c"),
          os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm", "-o", exe])
    r = _run([exe], env=dict(os.environ, **SAN_ENV), timeout=300)
    assert "0 mismatches" in r.stdout


def test_library_host_code_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    csrc = os.path.join(ROOT, "triangle_multiplication_amd", "csrc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", csrc]
    from triangle_multiplication_amd import build as lib_build
    srcs = list(lib_build.SOURCES)   # every source of libtrimul

    def build(src):
        obj = str(tmp_path / (src + ".o"))
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + inc +
             ["-x", "hip", "-c", os.path.join(csrc, src), "-o", obj] + HOST_SAN + ["-fno-gpu-sanitize"])
        return obj

    with cf.ThreadPoolExecutor(min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(build, srcs))
    drv = str(tmp_path / "driver.o")
    _run([HIPCC, "-O1", "-g"] + inc + ["-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-x", "c", "-c",
                                        os.path.join(ROOT, "tests", "sanitize", "host_driver.c"), "-o", drv] + HOST_SAN)
    exe = str(tmp_path / "host_san")
    _run([HIPCC, "--offload-arch=gfx950", "-o", exe, drv] + objs + HOST_SAN)
    work = tmp_path / "files"
    work.mkdir()
    r = _run([exe, str(work)], env=dict(os.environ, **SAN_ENV), timeout=300)
    assert "0 failures" in r.stdout
