import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: longer CPU test")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    # GPU tests never skip silently: on a machine without a GPU they are
    # deselected with -m "not gpu"; if selected, a missing GPU is a failure.
    if not gpu_available():
        pytest.fail("GPU test selected but no GPU is visible to torch")
    return True


@pytest.fixture(scope="session", autouse=True)
def built_library():
    """Build the HIP library if it is missing (it is not committed) or was
    built from other sources than the ones in the tree; a current build is
    used as it is."""
    from kv_cache_eviction_decode_amd.build import ensure_built
    ensure_built(verbose=True)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """One line per GPU parity run (tests/h2o_harness.py): heads and steps
    compared with the oracle, the largest output and score errors, the
    evictions checked, and the near-ties the oracle's margin excused. With
    H2O_PARITY_RECORD set, the same reports are written there as JSON."""
    import json
    import sys
    harness = sys.modules.get("h2o_harness")
    reports = getattr(harness, "REPORTS", None)
    if not reports:
        return
    tr = terminalreporter
    tr.section("GPU parity against the fp64 oracle")
    tr.write_line(f"{'run':34s} {'entry':22s} {'heads':>6s} {'steps':>5s} {'out err':>9s} {'score rel':>9s} "
                  f"{'colsum rel':>10s} {'evictions':>9s} {'exc.ev':>6s} {'exc.sel':>7s}")
    for r in reports:
        tr.write_line(f"{r.name[:34]:34s} {r.entry[:22]:22s} {r.heads:6d} {r.steps:5d} {r.max_out_err:9.2e} "
                      f"{r.max_score_rel:9.2e} {r.max_colsum_rel:10.2e} {r.evictions_checked:9d} "
                      f"{r.excused_evictions:6d} {r.excused_selections:7d}")
    path = os.environ.get("H2O_PARITY_RECORD")
    if path:
        with open(path, "w") as f:
            json.dump([r.as_dict() for r in reports], f, indent=1)
        tr.write_line(f"parity reports written to {path}")
