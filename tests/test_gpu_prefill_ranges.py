"""Prefill scoring on prompts whose scores jump far above everything before them.

The row pass of the 16-bit kernels keeps a fixed reference per query (the
maximum of the first key tile it sees) and only rescales when a tile's sum of
2^(c*s - reference) passes 2^64; the attention pass raises its reference when
a tile's maximum exceeds it by more than 8 (base 2). The generated workloads
never leave the fast paths, so these prompts place keys whose scores lie
16, 65 and 130 (base 2) above the first tile's: the first stays on the fast
path with terms near 2^16, the other two force the exact rescale. Column sums,
selected positions, the prompt's attention output and its normalisers are
compared with the fp64 oracle.
"""
import numpy as np
import pytest
import torch

from h2o_harness import SCORE_RTOL, TORCH_DTYPE, _rel_err, log, out_tolerance, to_device
from kv_cache_eviction_decode_amd import H2OCache
from oracle import H2OOracle
from oracle.h2o_oracle import prefill_attention

pytestmark = pytest.mark.gpu

MARGIN = 1e-5


def spiked_prompt(n, d, dtype, spikes, seed):
    """Queries 0.5 in every channel; keys small noise except the spiked rows,
    which hold a constant: score scale * 0.5 * value * d at those positions."""
    rng = np.random.default_rng(seed)
    Q = np.full((2, n, d), 0.5, np.float32)
    K = (0.1 * rng.standard_normal((2, n, d))).astype(np.float32)
    V = rng.standard_normal((2, n, d)).astype(np.float32)
    for pos, val in spikes:
        K[:, pos, :] = val
    cast = TORCH_DTYPE[dtype]
    rnd = lambda a: torch.from_numpy(a).to(cast).float().numpy()
    return rnd(Q), rnd(K), rnd(V)


CASES = [
    # name, dtype, d, n, spikes (position, key value)
    ("bf16_2wave", "bf16", 128, 700, [(300, 2.0), (500, 8.0), (650, 16.0)]),
    ("f16_2wave_d64", "f16", 64, 600, [(130, 4.0), (400, 16.0), (599, 32.0)]),
    ("bf16_4wave", "bf16", 128, 2300, [(700, 2.0), (1500, 8.0), (2100, 16.0)]),
    ("f16_4wave", "f16", 128, 2300, [(700, 2.0), (1500, 8.0), (2100, 16.0)]),
    # 10 blocks of 256: paired blocks (i, 9 - i) with a ragged last block
    ("bf16_4wave_paired", "bf16", 128, 2500, [(700, 2.0), (1500, 8.0), (2400, 16.0)]),
]


@pytest.mark.parametrize("mode", ["select", "attention"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_far_above_first_tile(gpu, case, mode):
    name, dtype, d, n, spikes = case
    log(f"[ranges] {name} mode={mode} n={n} d={d} spikes={spikes}")
    dev = torch.device("cuda:0")
    Q, K, V = spiked_prompt(n, d, dtype, spikes, seed=17)
    scale = d ** -0.5
    kh, kr = 24, 24
    cache = H2OCache(1, 2, d, kh, kr, TORCH_DTYPE[dtype], scale, dev)
    gQ, gK, gV = (to_device(x, dtype, dev).view(1, 2, n, d) for x in (Q, K, V))
    colsum = torch.empty(1, 2, n, dtype=torch.float32, device=dev)
    if mode == "attention":
        lse = torch.empty(1, 2, n, dtype=torch.float32, device=dev)
        out = cache.prefill_attention(gQ, gK, gV, lse_out=lse, colsum_out=colsum)
    else:
        cache.prefill_select(gQ, gK, gV, colsum_out=colsum)
    orc = H2OOracle(2, d, kh, kr, scale)
    pre = orc.prefill(Q, K, V)
    torch.cuda.synchronize()
    gcol = colsum.view(2, n).cpu().numpy()
    assert np.isfinite(gcol).all()
    rel = _rel_err(gcol, pre.colsum)
    assert rel.max() <= SCORE_RTOL, f"colsum rel err {rel.max():.3g}"
    # every row's probabilities sum to one, so the column sums add up to n
    assert abs(gcol.sum(axis=1) - n).max() <= 1e-4 * n
    gpos = cache.pos.view(2, -1).cpu().numpy()
    for g in range(2):
        if not np.array_equal(gpos[g], orc.pos[g]):
            assert pre.margin[g] < MARGIN, f"head {g}: selection differs, margin {pre.margin[g]:.3g}"
    if mode == "attention":
        gout = out.view(2, n, d).cpu().numpy()
        glse = lse.view(2, n).cpu().numpy()
        for g in range(2):
            ref_out, ref_lse = prefill_attention(Q[g], K[g], V[g], scale)
            err = float(np.abs(gout[g] - ref_out).max())
            assert err <= out_tolerance(dtype), f"head {g}: prompt output err {err:.3g}"
            lerr = float(np.abs(glse[g] - ref_lse).max())
            assert lerr <= 1e-4 * max(1.0, float(np.abs(ref_lse).max())), f"head {g}: lse err {lerr:.3g}"
    log(f"[ranges] {name} {mode}: colsum rel {rel.max():.2e}")
