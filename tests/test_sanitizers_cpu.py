"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Every source is rebuilt with the host side of each translation unit
instrumented (device code is not: the sanitizer flags are host-only), then
tests/abi_check.c and tests/test_abi_cpu.py run against that build. Neither
reaches a device call, so this runs without a GPU; any heap misuse or
undefined behaviour on the host paths (argument checks, sizes, descriptors,
error messages, state export) stops the run.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from kv_cache_eviction_decode_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]
ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
       "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}

pytestmark = pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not found")


@pytest.fixture(scope="module")
def sanitized_library(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("sanitized"))
    cc, digest = build.hipcc(), build.source_digest()

    def compile_one(src):
        obj = os.path.join(out, src.replace(".hip", ".o"))
        r = subprocess.run([cc, "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={build.ARCH}",
                            "-I", os.path.join(ROOT, "include"), *build.DEVICE_FLAGS, *HOST_SANITIZE,
                            f'-DH2O_SOURCE_DIGEST="{digest}"', "-c", os.path.join(build.CSRC, src), "-o", obj],
                           capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stderr
        return obj

    with ThreadPoolExecutor(len(build.SOURCES)) as ex:
        objs = list(ex.map(compile_one, build.SOURCES))
    lib = os.path.join(out, "libh2o.so")
    r = subprocess.run([cc, "-shared", "-fPIC", f"--offload-arch={build.ARCH}", *objs, *HOST_SANITIZE, "-o", lib],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr
    return lib


def test_c_abi_check_under_sanitizers(sanitized_library, tmp_path):
    exe = str(tmp_path / "abi_check")
    libdir = os.path.dirname(sanitized_library)
    r = subprocess.run([CLANG, "-std=c99", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_check.c"),
                        "-L", libdir, "-lh2o", "-Wl,-rpath," + libdir, "-o", exe],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env={**os.environ, **ENV})
    assert run.returncode == 0 and "abi_check ok" in run.stdout, run.stdout + run.stderr


def test_python_abi_tests_under_sanitizers(sanitized_library):
    runtime = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                             text=True).stdout.strip()
    assert os.path.exists(runtime), runtime
    env = {**os.environ, **ENV, "LD_PRELOAD": runtime, "H2O_LIBRARY": sanitized_library}
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                         capture_output=True, text=True, timeout=600, env=env, cwd=ROOT)
    assert run.returncode == 0, run.stdout[-3000:] + run.stderr[-3000:]
    assert "passed" in run.stdout and "AddressSanitizer" not in run.stderr + run.stdout
