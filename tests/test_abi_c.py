"""The C ABI from plain C: tests/abi_check.c is compiled as C99 against
include/h2o.h with gcc, linked to the built library and run (host-side paths
only, no GPU needed)."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "kv_cache_eviction_decode_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_is_c_and_abi_works_from_c():
    lib = os.path.join(PKG, "libh2o.so")
    assert os.path.exists(lib), "build the library first"
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "abi_check")
        cc = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                             "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_check.c"),
                             "-L", PKG, "-lh2o", "-Wl,-rpath," + PKG, "-o", exe],
                            capture_output=True, text=True, timeout=120)
        assert cc.returncode == 0, cc.stderr
        run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert run.returncode == 0, run.stderr + run.stdout
        assert "abi_check ok" in run.stdout


@pytest.mark.gpu
@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_caller_on_gpu(gpu):
    """tests/abi_gpu_check.c: init, prefill and decode driven from plain C
    (hipMalloc'd buffers, no PyTorch), checked against the zero-query closed form."""
    lib = os.path.join(PKG, "libh2o.so")
    assert os.path.exists(lib), "build the library first"
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "abi_gpu_check")
        cc = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                             "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                             os.path.join(ROOT, "tests", "abi_gpu_check.c"),
                             "-L", PKG, "-lh2o", "-Wl,-rpath," + PKG, "-L", "/opt/rocm/lib", "-lamdhip64",
                             "-Wl,-rpath,/opt/rocm/lib", "-lm", "-o", exe],
                            capture_output=True, text=True, timeout=120)
        assert cc.returncode == 0, cc.stderr
        run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert run.returncode == 0, run.stderr + run.stdout
        assert "abi_gpu_check ok" in run.stdout
