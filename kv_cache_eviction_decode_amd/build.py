"""Build step: compile the HIP sources for gfx950 into ``libh2o.so`` (in-tree).

Usage: ``python -m kv_cache_eviction_decode_amd.build``.

The library carries a digest of the sources it was built from (every file
under ``csrc/`` and ``include/h2o.h``): compiled in, returned by
``h2o_build_digest()``, and written beside the library as
``libh2o.so.digest``. ``ensure_built()`` rebuilds whenever that digest is
missing or differs from the sources' current one, and the binding refuses to
load a library whose compiled-in digest differs, so a test or benchmark can
never run a binary older than the sources next to it.
"""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libh2o.so")
SOURCES = ["api.hip", "decode.hip", "decode_split.hip", "decode_quant.hip", "prefill.hip"]

ARCH = "gfx950"
# Packed fp32 VALU ops (v_pk_*_f32) are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-I", os.path.join(ROOT, "include")]


def source_files(root: str = ROOT) -> list[str]:
    """Every file the library is built from: csrc/* and include/h2o.h, sorted."""
    csrc = os.path.join(root, "kv_cache_eviction_decode_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if os.path.isfile(os.path.join(csrc, f)))
    return files + [os.path.join(root, "include", "h2o.h")]


def source_digest(root: str = ROOT) -> str:
    """16 hex digits of SHA-256 over the names and contents of source_files(root)."""
    h = hashlib.sha256()
    for path in source_files(root):
        h.update(os.path.relpath(path, root).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()[:16]


def digest_path(lib: str = LIB) -> str:
    return lib + ".digest"


def built_digest(lib: str = LIB) -> str | None:
    """Digest recorded beside `lib` by the build that wrote it (None if absent)."""
    try:
        with open(digest_path(lib)) as f:
            return f.read().strip()
    except OSError:
        return None


def needs_build(root: str = ROOT, lib: str | None = None) -> bool:
    """True when the library is missing or was built from other sources."""
    lib = lib or os.path.join(root, "kv_cache_eviction_decode_amd", "libh2o.so")
    return not os.path.exists(lib) or built_digest(lib) != source_digest(root)


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    digest = source_digest()

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        _run([cc, *COMMON, *DEVICE_FLAGS, f'-DH2O_SOURCE_DIGEST="{digest}"', "-c", os.path.join(CSRC, src),
              "-o", obj])
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    with open(digest_path() + ".tmp", "w") as f:
        f.write(digest + "\n")
    os.replace(digest_path() + ".tmp", digest_path())
    if verbose:
        print(f"built {LIB} (sources {digest})")
    return LIB


def ensure_built(verbose: bool = False, root: str = ROOT, builder=None) -> bool:
    """Build unless the library next to the sources was built from exactly
    these sources. Returns True when a build ran."""
    if not needs_build(root):
        return False
    (builder or build)(verbose=verbose)
    return True


if __name__ == "__main__":
    build(verbose=True)
