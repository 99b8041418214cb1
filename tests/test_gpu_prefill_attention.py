"""GPU parity of the prefill entry points that share pass 1 with the model's
own prompt attention (h2o_prefill_attention) or take its normalisers
(h2o_prefill_select_lse), against the fp64 oracle, through the C ABI.

The prompt's attention output is compared element by element (max-abs 2e-2
for 16-bit inputs, 1e-4 for fp32) and its log normalisers to 1e-4 relative;
the column sums, the selection and the decode steps that follow must meet the
same bar as after h2o_prefill_select. Prompts span several 64-key tiles and
256-query blocks with ragged tails (fp32: several 64-row workgroups and
32-row streamed tiles), a single token, exactly one tile, both
head sizes and every input dtype; the named workloads run at full size with
sampled heads.
"""
import zlib

import pytest

from h2o_harness import ParityRun, log
from workload import WORKLOADS, Workload, sample_heads

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, H, d, dtype, n, k_heavy, k_recent, T
    ("ragged_bf16_d128", 2, 3, 128, "bf16", 300, 20, 20, 20),
    ("ragged_f16_d64", 1, 5, 64, "f16", 517, 33, 34, 20),
    ("f32_d128", 1, 2, 128, "f32", 129, 16, 33, 10),
    ("f32_d64", 2, 1, 64, "f32", 70, 8, 8, 10),
    ("f32_ragged_d128", 1, 3, 128, "f32", 461, 30, 30, 8),
    ("f32_long_d64", 2, 2, 64, "f32", 1000, 50, 50, 8),
    ("one_token_bf16", 2, 1, 128, "bf16", 1, 1, 1, 10),
    ("one_tile_f16", 1, 2, 128, "f16", 64, 12, 12, 10),
    ("two_blocks_bf16_d64", 1, 2, 64, "bf16", 600, 40, 40, 10),
    ("paired_blocks_bf16", 2, 3, 128, "bf16", 200, 20, 20, 10),  # blocks 0 and 1 in one workgroup
]


@pytest.mark.parametrize("mode", ["attention", "lse"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_modes_parity(gpu, case, mode):
    name, B, H, d, dt, n, kh, kr, T = case
    wl = Workload(name, B, H, d, dt, n, kh, kr, T, 1.5, 0.0, seed=zlib.crc32(name.encode()) % 10000)
    run = ParityRun(wl, T)
    run.prefill(mode=mode)
    rep = run.decode()
    log(f"[prefill {mode}] {name}: {rep}")
    assert rep.steps == T


def test_prefill_attention_u8_cache(gpu):
    wl = Workload("attn_u8", 1, 3, 128, "bf16", 333, 24, 24, 20, 1.5, 0.0, seed=77)
    run = ParityRun(wl, wl.steps, quant="u8")
    run.prefill(mode="attention")
    rep = run.decode()
    log(f"[prefill attention] u8 cache: {rep}")


@pytest.mark.parametrize("name,nsample", [("opt6.7b_layer", 8), ("opt30b_layer", 4), ("long_context", 2)])
def test_prefill_attention_full_size(gpu, name, nsample):
    wl = WORKLOADS[name]
    run = ParityRun(wl, 8, sample=sample_heads(wl, nsample), label=f"{name} {nsample} heads, attention prefill")
    run.prefill(mode="attention")
    rep = run.decode()
    log(f"[prefill attention] {name} full size: {rep}")
    assert rep.steps == 8


@pytest.mark.parametrize("dtype,n,batch", [("bf16", 1024, 64), ("f16", 2300, 16)])
def test_prefill_attention_zero_queries_closed_form(gpu, dtype, n, batch):
    """All-zero queries: every causal row is uniform, so the prompt's output row
    i is the running mean of V_0..V_i and its log normaliser is ln(i + 1); the
    column sums are harmonic differences. Checked on a sample of heads at the
    OPT-6.7B head count (2-wave prefill at n = 1024, 4-wave at 2300)."""
    import numpy as np
    import torch
    from h2o_harness import TORCH_DTYPE, to_device
    from kv_cache_eviction_decode_amd import H2OCache
    from workload import make_prompt, sample_heads
    wl = WORKLOADS["opt6.7b_layer"].with_(dtype=dtype, prompt_len=n, batch=batch)
    B, H, d = wl.batch, wl.heads, wl.head_dim
    dev = torch.device("cuda")
    sample = sample_heads(wl, 6)
    _, K, V = make_prompt(wl)
    cache = H2OCache(B, H, d, wl.k_heavy, wl.k_recent, TORCH_DTYPE[dtype], wl.scale, dev)
    lse = torch.empty(B, H, n, dtype=torch.float32, device=dev)
    colsum = torch.empty(B, H, n, dtype=torch.float32, device=dev)
    out = cache.prefill_attention(torch.zeros(B, H, n, d, dtype=TORCH_DTYPE[dtype], device=dev),
                                  to_device(K, dtype, dev).view(B, H, n, d), to_device(V, dtype, dev).view(B, H, n, d),
                                  lse_out=lse, colsum_out=colsum)
    idx = torch.from_numpy(sample).to(dev)
    gout = out.view(-1, n, d).index_select(0, idx).cpu().numpy()
    glse = lse.view(-1, n).index_select(0, idx).cpu().numpy()
    gcol = colsum.view(-1, n).index_select(0, idx).cpu().numpy()
    rows = np.arange(1, n + 1, dtype=np.float64)
    Hn = np.concatenate([[0.0], np.cumsum(1.0 / rows)])
    for j, g in enumerate(sample):
        mean = np.cumsum(V[g].astype(np.float64), axis=0) / rows[:, None]
        err = float(np.abs(gout[j] - mean).max())
        assert err <= 2e-2, f"head {g}: output err {err:.3g}"
        np.testing.assert_allclose(glse[j], np.log(rows), rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(gcol[j], Hn[n] - Hn[:n], rtol=1e-4)
    log(f"[attention] zero queries, {dtype} n={n}: closed form holds on {sample.size} heads")


# fp32 prompts with at least 1024 x 128 head rows take the two-rows-per-quad
# kernels (both head sizes); the GPU runs every head, the oracle checks a sample.
@pytest.mark.parametrize("case", [("f32_two_rows_d128", 4, 32, 128, 1030, "select"),
                                  ("f32_two_rows_d64", 8, 32, 64, 517, "select"),
                                  ("f32_two_rows_attention", 4, 32, 128, 1030, "attention")],
                         ids=lambda c: c[0])
def test_prefill_f32_two_rows(gpu, case):
    name, B, H, d, n, mode = case
    assert B * H * n >= 1024 * 128
    wl = Workload(name, B, H, d, "f32", n, 48, 48, 6, 1.5, 0.0, seed=zlib.crc32(name.encode()) % 10000)
    run = ParityRun(wl, wl.steps, sample=sample_heads(wl, 6), label=f"{name} 6 heads")
    run.prefill(mode=mode)
    rep = run.decode()
    log(f"[prefill {mode}] {name}: {rep}")
    assert rep.steps == wl.steps

