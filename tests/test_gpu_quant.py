"""GPU parity of the caches stored as 8-, 4- and 2-bit codes
(h2o_cache_init_quant) against the fp64 oracle's quantised modes, through the
C ABI.

Packed codes and grids of every cached row are compared bit for bit (both sides
take each rounding decision with the same fp32 operations); outputs, scores,
selections and evictions to the same tolerances as the plain cache. Cases
span both head sizes, every input dtype, ragged prompts, a cache still
filling, a one-token prompt (degenerate key grids), every policy, a sink
token, and the OPT-6.7B layer at full size.
"""
import zlib

import pytest
import torch

from h2o_harness import ParityRun, log
from workload import WORKLOADS, Workload, sample_heads

pytestmark = pytest.mark.gpu

QUANT_CASES = [
    # name, policy, B, H, d, dtype, n, k_heavy, k_recent, T, sink
    ("ragged_bf16", "accumulated", 2, 3, 128, "bf16", 300, 20, 20, 60, 0.0),
    ("f16_d64", "accumulated", 1, 5, 64, "f16", 517, 33, 34, 40, 0.0),
    ("fills_bf16_d64", "accumulated", 1, 3, 64, "bf16", 20, 24, 24, 50, 0.0),
    ("f32_d128", "accumulated", 1, 2, 128, "f32", 129, 16, 33, 30, 0.0),
    ("one_token_prompt", "accumulated", 2, 1, 128, "bf16", 1, 1, 1, 20, 0.0),
    ("heavy_only", "accumulated", 1, 2, 128, "bf16", 300, 32, 0, 40, 0.0),
    ("averaged_f16", "averaged", 1, 2, 128, "f16", 200, 24, 24, 40, 0.0),
    ("position_bf16", "position", 2, 2, 64, "bf16", 333, 4, 28, 40, 0.0),
    ("sink_f16", "accumulated", 1, 2, 128, "f16", 2048, 205, 205, 16, 4.0),
]


FORMATS = ["u8", "u4", "u2"]


@pytest.mark.parametrize("quant", FORMATS)
@pytest.mark.parametrize("case", QUANT_CASES, ids=[c[0] for c in QUANT_CASES])
def test_quant_parity(gpu, case, quant):
    name, policy, B, H, d, dt, n, kh, kr, T, sink = case
    wl = Workload(f"{quant}_" + name, B, H, d, dt, n, kh, kr, T, 1.5, sink,
                  seed=zlib.crc32(name.encode()) % 10000)
    run = ParityRun(wl, T, policy=policy, quant=quant)
    run.prefill()
    rep = run.decode()
    log(f"[{quant}] {name} ({policy}): {rep}")
    assert rep.steps == T


@pytest.mark.parametrize("quant", FORMATS)
def test_quant_opt_layer_full_size(gpu, quant):
    """The OPT-6.7B layer shape (2048 heads x 256 slots), as in the benchmark:
    32 heads over all 512 decode steps."""
    wl = WORKLOADS["opt6.7b_layer"]
    run = ParityRun(wl, wl.steps, sample=sample_heads(wl, 32), quant=quant,
                    label=f"opt6.7b_layer 32 heads x all steps")
    run.prefill()
    rep = run.decode()
    log(f"[{quant}] opt6.7b_layer full size: {rep}")
    assert rep.steps == wl.steps


@pytest.mark.parametrize("quant", FORMATS)
def test_quant_wave_kernel_beyond_prefetch(gpu, quant):
    """1024 heads (one wave per head) with 320 slots: the scores and positions
    past the 256 prefetched per head are read in the epilogue."""
    wl = Workload("quant_wave_320", 32, 32, 128, "bf16", 400, 160, 160, 10, 1.5, 0.0, 91)
    run = ParityRun(wl, wl.steps, sample=sample_heads(wl, 8), quant=quant)
    run.prefill()
    rep = run.decode()
    log(f"[{quant}] wave kernel, 320 slots: {rep}")
    assert rep.steps == wl.steps


@pytest.mark.parametrize("quant", FORMATS)
def test_quant_wave_kernel_filling(gpu, quant):
    """1024 heads (one wave per head) whose cache fills during decode: a
    100-token prompt into 161 slots, so the occupied count (100 to 161) ends
    inside a batch of rows at every step and the rows past it must read as
    nothing, then 9 steps with the cache full."""
    wl = Workload("quant_wave_filling", 32, 32, 128, "bf16", 100, 81, 80, 70, 1.5, 0.0, 57)
    run = ParityRun(wl, wl.steps, sample=sample_heads(wl, 8), quant=quant)
    run.prefill()
    rep = run.decode()
    log(f"[{quant}] wave kernel, cache filling: {rep}")
    assert rep.steps == wl.steps


@pytest.mark.parametrize("quant", FORMATS)
def test_quant_max_slots(gpu, quant):
    """The largest cache, 8192 slots of codes, for two heads (the
    workgroup-per-head kernel) over 4 steps with the cache full."""
    wl = Workload("quant_max_slots", 1, 2, 128, "bf16", 8300, 4096, 4096, 4, 1.5, 0.0, 35)
    run = ParityRun(wl, wl.steps, quant=quant)
    run.prefill()
    rep = run.decode()
    log(f"[{quant}] max slots, 2 heads: {rep}")
    assert rep.steps == wl.steps


def test_quant_max_slots_wave_kernel(gpu):
    """8192 slots of 4-bit codes for 1024 heads (the one-wave-per-head
    kernel, 32 KiB of logits in LDS); 4 sampled heads over 4 steps."""
    wl = Workload("quant_max_slots_1024", 8, 128, 128, "bf16", 8300, 4096, 4096, 4, 1.5, 0.0, 36)
    run = ParityRun(wl, wl.steps, sample=sample_heads(wl, 4), quant="u4")
    run.prefill()
    rep = run.decode()
    log(f"[u4] max slots, 1024 heads: {rep}")
    assert rep.steps == wl.steps


@pytest.mark.parametrize("quant", FORMATS)
def test_quant_uniform_closed_form_full_shape(gpu, quant):
    """All-zero queries at the OPT-6.7B layer shape over a cache of codes:
    every logit is 0 whatever the key codes, so the column sums are harmonic
    differences, the selection is the first k_heavy plus the window, and every
    step evicts t - k_recent. Each output is the mean of the cached values as
    stored, so it lies within the largest half grid step of its rows of the
    mean of the exact values (the new token attends at full precision)."""
    import numpy as np
    from h2o_harness import to_device
    from kv_cache_eviction_decode_amd import H2OCache
    from workload import make_decode, make_prompt
    wl = WORKLOADS["opt6.7b_layer"]
    B, H, d, n, kh, kr = wl.batch, wl.heads, wl.head_dim, wl.prompt_len, wl.k_heavy, wl.k_recent
    T = 16
    levels = {"u8": 255, "u4": 15, "u2": 3}[quant]
    dev = torch.device("cuda")
    _, K, V = make_prompt(wl)
    _, kd, vd = make_decode(wl, steps=T)
    cache = H2OCache(B, H, d, kh, kr, torch.bfloat16, wl.scale, dev, quant=quant)
    Qz = torch.zeros(B, H, n, d, dtype=torch.bfloat16, device=dev)
    colsum = torch.empty(B, H, n, dtype=torch.float32, device=dev)
    cache.prefill_select(Qz, to_device(K, "bf16", dev).view(B, H, n, d), to_device(V, "bf16", dev).view(B, H, n, d),
                         colsum_out=colsum)
    Hn = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1))])
    np.testing.assert_allclose(colsum.cpu().numpy().reshape(-1, n), np.broadcast_to(Hn[n] - Hn[:n], (B * H, n)),
                               rtol=1e-4)
    expect = np.array(list(range(kh)) + list(range(n - kr, n)), dtype=np.int32)
    assert (cache.pos.cpu().numpy().reshape(-1, wl.k) == expect).all()
    allv = np.concatenate([V, vd], axis=1).astype(np.float64)  # [G, n+T, d]
    half_step = (allv.max(axis=2) - allv.min(axis=2)) / levels / 2  # per row
    members = np.broadcast_to(expect, (B * H, wl.k)).copy()
    qz = torch.zeros(B, H, d, dtype=torch.bfloat16, device=dev)
    kdg = to_device(kd.transpose(1, 0, 2), "bf16", dev).view(T, B, H, d)
    vdg = to_device(vd.transpose(1, 0, 2), "bf16", dev).view(T, B, H, d)
    for t in range(T):
        out, ev = cache.decode_step(qz, kdg[t], vdg[t])
        pos_t = n + t
        assert (ev.cpu().numpy() == pos_t - kr).all(), f"step {t}"
        idx = np.concatenate([members, np.full((B * H, 1), pos_t)], axis=1)
        mean = np.take_along_axis(allv, idx[:, :, None], axis=1).mean(axis=1)
        bound = np.take_along_axis(half_step, members, axis=1).max(axis=1) + 1e-5
        err = np.abs(out.cpu().numpy().reshape(B * H, d) - mean).max(axis=1)
        assert (err <= bound).all(), f"step {t}: {err.max()} > {bound[err.argmax()]}"
        members[members == pos_t - kr] = pos_t
    log(f"[{quant}] uniform closed form at full shape: {T} steps")


@pytest.mark.parametrize("quant", FORMATS)
def test_quant_errors(gpu, quant):
    from kv_cache_eviction_decode_amd import H2OCache, binding as b
    c = H2OCache(1, 2, 128, 8, 8, torch.bfloat16, device="cuda", quant=quant)
    z = torch.zeros(1, 2, 0, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(b.H2OError, match="at least one token"):
        c.prefill_select(z, z, z)
    q = torch.zeros(1, 2, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(b.H2OError, match="split decode"):
        c.decode_step_split(q, q, q)
    assert c.t_next == 0
