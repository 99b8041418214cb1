"""The hand-worked examples of tests/golden/ run on the GPU path.

Each example's one- or two-channel queries, keys and values sit in the
first channels of d = 64 vectors (the rest zero, which changes no dot
product), in fp32, with the example's scale. The GPU's column sums, kept
positions, scores, evictions and outputs are compared with the fractions
worked out by hand (fp32 tolerance), not with the oracle.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from h2o_harness import log
from kv_cache_eviction_decode_amd import H2OCache

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D = 64
RTOL = 1e-5


def _load(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = (x.strip() for x in line.split("=", 1))
                vals[k] = v
    return vals


def _fr(s):
    return np.array([float(Fraction(x)) for x in s.split()])


def _inputs(g):
    n, d, steps = int(g["n"]), int(g["d"]), int(g["steps"])
    N = n + steps
    q = np.zeros((N, D), np.float32)
    k = np.zeros((N, D), np.float32)
    v = np.zeros((N, D), np.float32)
    if g.get("query") == "zero":
        k[:, :d] = 1.0
        scale = 1.0 / np.sqrt(d)
    else:
        q[:, 0] = 1.0
        w = [float(x) for x in (g["prompt_weights"] + " " + g["decode_weights"]).split()]
        k[:, 0] = np.log(np.array(w, np.float64)).astype(np.float32)
        scale = 1.0
    v[:, 0] = np.arange(N, dtype=np.float32)
    if g["value"] == "position_and_one":
        v[:, 1] = 1.0
    return n, d, steps, q, k, v, scale


@pytest.mark.parametrize("name", ["illustration_budget3.txt", "weighted_budget3.txt", "averaged_budget3.txt",
                                  "heavy_only_budget2.txt"])
def test_golden_on_gpu(gpu, name):
    g = _load(name)
    n, d, steps, q, k, v, scale = _inputs(g)
    log(f"[golden-gpu] {name}")
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    cache = H2OCache(1, 1, D, int(g["k_heavy"]), int(g["k_recent"]), torch.float32, scale, dev,
                     policy=g.get("policy", "accumulated"))
    colsum = torch.empty(1, 1, n, dtype=torch.float32, device=dev)
    cache.prefill_select(t(q[:n]).view(1, 1, n, D), t(k[:n]).view(1, 1, n, D), t(v[:n]).view(1, 1, n, D),
                         colsum_out=colsum)
    torch.cuda.synchronize()
    np.testing.assert_allclose(colsum.view(-1).cpu().numpy(), _fr(g["colsum"]), rtol=RTOL)
    assert cache.pos.view(-1).tolist() == [int(x) for x in g["after_prefill_pos"].split()]
    np.testing.assert_allclose(cache.score.view(-1).cpu().numpy(), _fr(g["after_prefill_score"]), rtol=RTOL)
    for s in range(steps):
        i = n + s
        out, ev = cache.decode_step(t(q[i]).view(1, 1, D), t(k[i]).view(1, 1, D), t(v[i]).view(1, 1, D))
        torch.cuda.synchronize()
        assert int(ev.item()) == int(g[f"step{s}_evicted"]), f"step {s}"
        want = _fr(g[f"step{s}_out"])
        got = out.view(-1).cpu().numpy()
        np.testing.assert_allclose(got[:want.size], want, rtol=RTOL)
        assert np.all(got[want.size:] == 0.0)
    assert cache.pos.view(-1).tolist() == [int(x) for x in g["final_pos"].split()]
    np.testing.assert_allclose(cache.score.view(-1).cpu().numpy(), _fr(g["final_score"]), rtol=RTOL)
