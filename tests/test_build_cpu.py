"""The library that tests, smoke() and the benchmark load is always built from
the sources beside it (CPU only): a source edit makes the build stale, the
build helper then rebuilds, and the binding refuses a stale binary."""
import os
import shutil
import subprocess
import sys

from kv_cache_eviction_decode_amd import binding, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _copy_tree(dst, with_library=False):
    pkg = os.path.join(dst, "kv_cache_eviction_decode_amd")
    shutil.copytree(build.CSRC, os.path.join(pkg, "csrc"))
    os.makedirs(os.path.join(dst, "include"))
    shutil.copy(binding.HEADER, os.path.join(dst, "include", "h2o.h"))
    if with_library:
        for f in ("__init__.py", "binding.py", "build.py", "libh2o.so"):
            shutil.copy(os.path.join(build.PKG, f), os.path.join(pkg, f))
    return pkg


def test_in_tree_library_matches_sources():
    lib = binding.load_library()
    assert lib.h2o_build_digest().decode() == build.source_digest() == build.built_digest()
    assert not build.needs_build()


def test_source_edit_triggers_rebuild(tmp_path):
    root = str(tmp_path)
    pkg = _copy_tree(root)
    lib = os.path.join(pkg, "libh2o.so")
    with open(lib, "wb") as f:
        f.write(b"stand-in")
    with open(build.digest_path(lib), "w") as f:
        f.write(build.source_digest(root) + "\n")
    calls = []
    assert not build.needs_build(root)
    assert build.ensure_built(root=root, builder=lambda verbose: calls.append(1)) is False and calls == []

    with open(os.path.join(pkg, "csrc", "decode.hip"), "a") as f:
        f.write("\n// edited\n")
    assert build.source_digest(root) != build.source_digest(ROOT)
    assert build.needs_build(root)
    assert build.ensure_built(root=root, builder=lambda verbose: calls.append(1)) is True and calls == [1]

    os.remove(build.digest_path(lib))  # a build that recorded nothing is stale too
    with open(os.path.join(pkg, "csrc", "decode.hip"), "w") as f:
        f.write(open(os.path.join(build.CSRC, "decode.hip")).read())
    assert build.needs_build(root)


def test_header_edit_changes_the_digest(tmp_path):
    root = str(tmp_path)
    _copy_tree(root)
    before = build.source_digest(root)
    assert before == build.source_digest(ROOT)
    with open(os.path.join(root, "include", "h2o.h"), "a") as f:
        f.write("\n/* edited */\n")
    assert build.source_digest(root) != before


def test_stale_library_is_refused_at_load(tmp_path):
    root = str(tmp_path)
    pkg = _copy_tree(root, with_library=True)
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from kv_cache_eviction_decode_amd import binding\n"
            "try:\n"
            "    binding.load_library()\n"
            "except ImportError as e:\n"
            "    print('refused', e)\n"
            "else:\n"
            "    print('loaded')\n") % root
    run = lambda: subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                                 cwd=root)
    r = run()
    assert r.returncode == 0 and "loaded" in r.stdout, r.stdout + r.stderr
    with open(os.path.join(pkg, "csrc", "prefill.hip"), "a") as f:
        f.write("\n// edited\n")
    r = run()
    assert r.returncode == 0 and "refused" in r.stdout and "built from sources" in r.stdout, r.stdout + r.stderr
