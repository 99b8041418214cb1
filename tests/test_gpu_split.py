"""GPU parity of the split decode entry point (h2o_decode_step_split) against
the fp64 oracle, through the C ABI.

Chunk lengths are chosen so that heads have one chunk, a few, a ragged last
chunk, more than 64 chunks (the merge loops over lane-sized groups of
partials) and an empty chunk (empty cache). The cache grows through chunk
boundaries while it fills. A few-heads shape (one sequence of eight heads) runs with
the library's own chunking, as in the benchmark; the long-context workload
at full size, over every decode step, is in tests/test_gpu_parity.py.
"""
import zlib

import pytest
import torch

from h2o_harness import ParityRun, log
from workload import WORKLOADS, Workload, sample_heads

pytestmark = pytest.mark.gpu

SPLIT_CASES = [
    # name, policy, B, H, d, dtype, n, k_heavy, k_recent, T, chunk_rows
    ("ragged_chunks_bf16", "accumulated", 1, 3, 128, "bf16", 700, 150, 150, 30, 64),
    ("fills_across_chunks_f16_d64", "accumulated", 1, 2, 64, "f16", 100, 100, 100, 120, 64),
    ("auto_chunks_f32", "accumulated", 2, 2, 128, "f32", 900, 200, 100, 20, 0),
    ("one_chunk_bf16", "accumulated", 2, 2, 128, "bf16", 300, 40, 40, 30, 128),
    ("empty_prompt_bf16", "accumulated", 1, 2, 128, "bf16", 0, 40, 40, 100, 64),
    ("heavy_only_bf16", "accumulated", 1, 2, 128, "bf16", 500, 256, 0, 30, 128),
    ("averaged_bf16_d64", "averaged", 1, 2, 64, "bf16", 600, 128, 64, 30, 64),
    ("position_f16", "position", 1, 2, 128, "f16", 400, 8, 120, 30, 64),
    ("many_chunks_bf16", "accumulated", 1, 1, 128, "bf16", 9000, 4096, 4096, 4, 64),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_split_parity(gpu, case):
    name, policy, B, H, d, dt, n, kh, kr, T, rows = case
    wl = Workload(name, B, H, d, dt, n, kh, kr, T, 1.5, 0.0, seed=zlib.crc32(name.encode()) % 10000)
    run = ParityRun(wl, T, policy=policy, split_rows=rows)
    run.prefill()
    rep = run.decode()
    log(f"[split] {name} ({policy}, chunk_rows={rows}): {rep}")
    assert rep.steps == T


def test_split_few_heads_auto_chunks(gpu):
    """Eight heads of 2048 slots: the library cuts each into 32 chunks."""
    wl = WORKLOADS["long_context"].with_(batch=1, heads=8, prompt_len=4096, steps=40)
    run = ParityRun(wl, wl.steps, split_rows=0)
    run.prefill()
    rep = run.decode()
    log(f"[split] few heads: {rep}")
    assert rep.steps == wl.steps


def test_split_errors(gpu):
    from kv_cache_eviction_decode_amd import H2OCache, binding as b
    c = H2OCache(1, 2, 128, 8, 8, torch.bfloat16, device="cuda")
    q = torch.zeros(1, 2, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(1, 2, 128, dtype=torch.float32, device="cuda")
    ev = torch.empty(1, 2, dtype=torch.int32, device="cuda")
    small = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(b.H2OError, match="H2O_EWORKSPACE"):
        b.h2o_decode_step_split(c.desc, q, q, q, out, ev, small, 0)
    with pytest.raises(b.H2OError, match="multiple of 64"):
        b.h2o_decode_step_split(c.desc, q, q, q, out, ev, c.split_workspace(), 100)
    assert c.t_next == 0  # rejected calls change nothing
    c.decode_step_split(q, q, q, out, ev)
    torch.cuda.synchronize()
    assert c.t_next == 1 and ev.tolist() == [[-1, -1]]


def test_split_uniform_closed_form(gpu):
    """All-zero queries through the split entry point at the long-context shape
    with one sequence (32 heads x 2048 slots, the library's chunking): column
    sums are harmonic differences, the selection is the first k_heavy tokens
    plus the window, every step evicts t - k_recent and each output is the
    plain mean of the cached values and the new one."""
    import numpy as np
    from h2o_harness import to_device
    from kv_cache_eviction_decode_amd import H2OCache
    from workload import make_decode, make_prompt
    wl = WORKLOADS["long_context"].with_(batch=1)
    B, H, d, n, kh, kr = wl.batch, wl.heads, wl.head_dim, wl.prompt_len, wl.k_heavy, wl.k_recent
    T = 8
    dev = torch.device("cuda")
    _, K, V = make_prompt(wl)
    _, kd, vd = make_decode(wl, steps=T)
    cache = H2OCache(B, H, d, kh, kr, torch.bfloat16, wl.scale, dev)
    colsum = torch.empty(B, H, n, dtype=torch.float32, device=dev)
    cache.prefill_select(torch.zeros(B, H, n, d, dtype=torch.bfloat16, device=dev),
                         to_device(K, "bf16", dev).view(B, H, n, d), to_device(V, "bf16", dev).view(B, H, n, d),
                         colsum_out=colsum)
    Hn = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1))])
    np.testing.assert_allclose(colsum.cpu().numpy().reshape(-1, n), np.broadcast_to(Hn[n] - Hn[:n], (B * H, n)),
                               rtol=1e-4)
    expect = np.array(list(range(kh)) + list(range(n - kr, n)), dtype=np.int32)
    assert (cache.pos.cpu().numpy().reshape(-1, wl.k) == expect).all()
    allv = np.concatenate([V, vd], axis=1).astype(np.float64)
    members = np.broadcast_to(expect, (B * H, wl.k)).copy()
    qz = torch.zeros(B, H, d, dtype=torch.bfloat16, device=dev)
    kdg = to_device(kd.transpose(1, 0, 2), "bf16", dev).view(T, B, H, d)
    vdg = to_device(vd.transpose(1, 0, 2), "bf16", dev).view(T, B, H, d)
    for t in range(T):
        out, ev = cache.decode_step_split(qz, kdg[t], vdg[t])
        pos_t = n + t
        assert (ev.cpu().numpy() == pos_t - kr).all(), f"step {t}"
        idx = np.concatenate([members, np.full((B * H, 1), pos_t)], axis=1)
        mean = np.take_along_axis(allv, idx[:, :, None], axis=1).mean(axis=1)
        err = np.abs(out.cpu().numpy().reshape(B * H, d) - mean).max()
        assert err <= 1e-5, f"step {t}: {err}"
        members[members == pos_t - kr] = pos_t
    log(f"[split] uniform closed form, 32 heads x {wl.k} slots: {T} steps")
