"""The C-ABI library loads on a machine without a GPU, exports every declared
entry point, and rejects bad arguments before touching the device (CPU only)."""
import ctypes
import os
import re

import pytest

from kv_cache_eviction_decode_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(b.HEADER) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(h2o_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = b.load_library()
    names = _declared_functions()
    assert set(names) >= {"h2o_prefill_select", "h2o_decode_step", "h2o_cache_state"}
    for name in names:
        assert hasattr(lib, name), name
    # every declared function has a binding with the same name
    for name in names:
        assert callable(getattr(b, name)), name


def test_workspace_bytes():
    ws = b.h2o_prefill_workspace_bytes
    assert ws(64, 32, 1024) == 2 * 64 * 32 * 1024 * 4
    assert ws(1, 1, 1) == 256 + 256  # lse rows padded to 64 floats, regions 256-byte aligned
    assert ws(0, 4, 10) == 0 and ws(1, 1, -1) == 0
    assert ws(8, 32, 16384) == 2 * 8 * 32 * 16384 * 4


def test_decode_workspace_bytes():
    ws = b.h2o_decode_workspace_bytes
    # logits [k], ceil(k/64) partials of (max, sum) and d accumulators, 256-byte aligned regions
    assert ws(1, 1, 128, 2048) == 8192 + 256 + 32 * 128 * 4
    assert ws(8, 32, 128, 2048) == 256 * 2048 * 4 + 256 * 32 * 2 * 4 + 256 * 32 * 128 * 4
    assert ws(1, 1, 64, 65) == 512 + 256 + 512
    assert ws(1, 1, 96, 64) == 0 and ws(1, 1, 128, 0) == 0 and ws(1, 1, 128, 8193) == 0


def test_struct_layout_matches_header():
    # the descriptor is a plain C struct: 8 x 4-byte fields, 4 pointers, 2 int32, int64, 2 x 4 bytes, 2 pointers
    assert ctypes.sizeof(b.h2o_cache) == 8 * 4 + 4 * 8 + 2 * 4 + 8 + 2 * 4 + 2 * 8
    assert b.h2o_cache.K.offset == 32 and b.h2o_cache.steps.offset == 72
    assert b.h2o_cache.quant.offset == 84 and b.h2o_cache.k_qparam.offset == 88
    assert ctypes.sizeof(b.h2o_state) == 32


@pytest.mark.parametrize("args,msg", [
    ((1, 1, 96, 1, 1, 0, 1, 0.1), "head_dim"),
    ((1, 1, 128, 1, -1, 0, 1, 0.1), "k_recent"),
    ((1, 1, 128, 0, 0, 0, 1, 0.1), "k = k_heavy + k_recent must be >= 1"),
    ((1, 1, 128, -1, 1, 0, 1, 0.1), "k_heavy"),
    ((0, 1, 128, 1, 1, 0, 1, 0.1), "batch"),
    ((1, 1, 128, 8192, 1, 0, 1, 0.1), "exceeds"),
    ((1, 1, 128, 1, 1, 0, 7, 0.1), "dtype"),
    ((1, 1, 128, 1, 1, 3, 1, 0.1), "policy"),
    ((1, 1, 128, 1, 1, 0, 1, float("nan")), "scale"),
    ((1, 1, 128, 1, 1, 0, 1, 0.1), "non-NULL"),
    ((1, 1, 128, 4, 0, 2, 1, 0.1), "non-NULL"),
])
def test_init_rejects_bad_arguments_without_launching(args, msg):
    lib = b.load_library()
    d = b.h2o_cache()
    st = lib.h2o_cache_init(ctypes.byref(d), *args, None, None, None, None, None)
    assert st == b.H2O_EINVAL
    assert msg in b.h2o_last_error()
    assert d.magic == 0  # descriptor untouched


@pytest.mark.parametrize("quant", [b.H2O_QUANT_U8, b.H2O_QUANT_U4, b.H2O_QUANT_U2])
def test_quant_init_rejects_missing_grids(quant):
    lib = b.load_library()
    d = b.h2o_cache()
    st = lib.h2o_cache_init_quant(ctypes.byref(d), 1, 1, 128, 4, 4, 0, 1, 0.1, quant, None, None, None, None,
                                  None, None, None)
    assert st == b.H2O_EINVAL and "k_qparam" in b.h2o_last_error() and d.magic == 0


@pytest.mark.parametrize("quant", [b.H2O_QUANT_NONE, 4, -1])
def test_quant_init_rejects_unknown_format(quant):
    lib = b.load_library()
    d = b.h2o_cache()
    st = lib.h2o_cache_init_quant(ctypes.byref(d), 1, 1, 128, 4, 4, 0, 1, 0.1, quant, None, None, None, None,
                                  None, None, None)
    assert st == b.H2O_EINVAL and "code format" in b.h2o_last_error() and d.magic == 0


def test_quant_constants_match_header():
    import re
    text = open(b.HEADER).read()
    vals = {m.group(1): int(m.group(2)) for m in re.finditer(r"(H2O_QUANT_\w+)\s*=\s*(\d+)", text)}
    assert vals == {"H2O_QUANT_NONE": b.H2O_QUANT_NONE, "H2O_QUANT_U8": b.H2O_QUANT_U8,
                    "H2O_QUANT_U4": b.H2O_QUANT_U4, "H2O_QUANT_U2": b.H2O_QUANT_U2}


def test_calls_on_uninitialised_cache_are_rejected():
    lib = b.load_library()
    d = b.h2o_cache()
    st_ = b.h2o_state()
    assert lib.h2o_decode_step(ctypes.byref(d), None, None, None, None, None, None) == b.H2O_ESTATE
    assert lib.h2o_prefill_select(ctypes.byref(d), None, None, None, 4, None, 0, None, None) == b.H2O_ESTATE
    assert lib.h2o_cache_state(ctypes.byref(d), ctypes.byref(st_), None, None, None) == b.H2O_ESTATE
    assert lib.h2o_cache_restore(ctypes.byref(d), 3, 0) == b.H2O_ESTATE
    assert lib.h2o_decode_step_split(ctypes.byref(d), None, None, None, None, None, 0, None, 0, None) == b.H2O_ESTATE
    assert lib.h2o_decode_step(None, None, None, None, None, None, None) == b.H2O_EINVAL


def test_noalloc_split_rejects_before_launching():
    """The allocation-free split step checks the cache and its workspace need
    against the library's own array before any device call."""
    lib = b.load_library()
    d = b.h2o_cache()
    assert lib.h2o_decode_step_split_noalloc(ctypes.byref(d), None, None, None, None, None, 0, None) == b.H2O_ESTATE
    assert lib.h2o_decode_step_split_noalloc(None, None, None, None, None, None, 0, None) == b.H2O_EINVAL
    # a descriptor as h2o_cache_init would leave it, for 256 heads x 8192 slots: 24 MiB of workspace
    big = b.h2o_cache(batch=8, heads=32, head_dim=128, k_heavy=4096, k_recent=4096, magic=0x48324F31)
    need = b.h2o_decode_workspace_bytes(8, 32, 128, 8192)
    assert need > b.H2O_SPLIT_SCRATCH_BYTES
    st = lib.h2o_decode_step_split_noalloc(ctypes.byref(big), None, None, None, None, None, 0, None)
    assert st == b.H2O_EWORKSPACE and str(need) in b.h2o_last_error()


def test_scratch_size_matches_header():
    text = open(b.HEADER).read()
    m = re.search(r"#define\s+H2O_SPLIT_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == b.H2O_SPLIT_SCRATCH_BYTES


def test_fullcache_rejects_bad_arguments():
    lib = b.load_library()
    assert lib.h2o_fullcache_decode(1, 1, 128, 1, 0.1, 0, None, None, None, None, None) == b.H2O_EINVAL
    assert "len" in b.h2o_last_error()
    assert lib.h2o_fullcache_decode(1, 1, 100, 1, 0.1, 4, None, None, None, None, None) == b.H2O_EINVAL


def test_raised_error_carries_library_message():
    with pytest.raises(b.H2OError, match="H2O_ESTATE"):
        b.h2o_cache_restore(b.h2o_cache(), 1)


def test_missing_library_fails_loudly():
    """Without the built HIP library the binding raises; there is no fallback path."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from kv_cache_eviction_decode_amd import binding\n"
            "try:\n"
            "    binding.load_library('/nonexistent/libh2o.so')\n"
            "except ImportError as e:\n"
            "    print('raised', e)\n"
            "else:\n"
            "    sys.exit(3)\n") % ROOT
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "raised" in r.stdout


def test_package_does_not_import_the_oracle():
    """The product package never loads the test oracle."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import kv_cache_eviction_decode_amd\n"
            "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')]\n"
            "sys.exit(1 if bad else 0)\n") % ROOT
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr


def test_build_compiles_every_kernel_source():
    """Every .hip file of the package is part of the library build."""
    import glob
    from kv_cache_eviction_decode_amd import build
    on_disk = sorted(os.path.basename(p) for p in glob.glob(os.path.join(build.CSRC, "*.hip")))
    assert on_disk == sorted(build.SOURCES)
