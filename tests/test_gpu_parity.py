"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Small cases run the oracle on every head; they span several prefill tiles,
ragged tails, empty and tiny prompts, prompts shorter than the cache,
k_heavy = 0, the largest k, every dtype and both head sizes. The named
workloads run at their full shapes (same grid as the benchmark) over every
decode step: every head of the OPT-6.7B, OPT-30B and long-context layers
(the last with the fused and with the split entry point), and 512 of the
large-batch layer's 8192 heads, whose every head is also checked over the
first four steps.
"""
import zlib

import numpy as np
import pytest
import torch

from h2o_harness import TORCH_DTYPE, ParityRun, log, out_tolerance, to_device
from workload import WORKLOADS, Workload, make_decode, make_prompt, sample_heads

pytestmark = pytest.mark.gpu

SMALL = [
    # name, B, H, d, dtype, n, k_heavy, k_recent, T, alpha, sink
    ("ragged_bf16_d128", 2, 3, 128, "bf16", 300, 20, 20, 60, 1.5, 0.0),
    ("ragged_f16_d64", 1, 5, 64, "f16", 517, 33, 34, 40, 1.5, 0.0),
    ("fills_bf16_d64", 1, 3, 64, "bf16", 20, 24, 24, 50, 1.5, 0.0),
    ("local_only_f32_d128", 1, 2, 128, "f32", 129, 0, 33, 30, 1.5, 0.0),
    ("empty_prompt_bf16", 1, 2, 128, "bf16", 0, 8, 8, 40, 1.5, 0.0),
    ("one_token_bf16", 2, 1, 128, "bf16", 1, 1, 1, 20, 1.5, 0.0),
    ("n_eq_k_plus_1_f16", 1, 2, 128, "f16", 65, 32, 32, 10, 1.5, 0.0),
    ("sink_f16_d128", 1, 2, 128, "f16", 2048, 205, 205, 16, 1.5, 4.0),
    ("f32_d64_odd_k", 2, 2, 64, "f32", 200, 7, 6, 30, 1.2, 0.0),
    ("bf16_long_tail", 1, 1, 128, "bf16", 1500, 100, 1, 24, 1.2, 0.0),
    # prompts over 2048 tokens take 4-wave workgroups; a ragged last block
    # leaves whole waves past the prompt (2100) or one wave partly inside (2500)
    ("ragged_4wave_bf16", 1, 2, 128, "bf16", 2100, 64, 64, 8, 1.5, 0.0),
    ("ragged_4wave_f16_d64", 1, 1, 64, "f16", 2500, 30, 31, 6, 1.2, 0.0),
    # whole 64-row tiles, but not whole workgroups: the last workgroup's later
    # waves lie past the prompt while its last tile is full
    ("tile_multiple_2wave_f16_d64", 1, 2, 64, "f16", 192, 32, 32, 8, 1.5, 0.0),
    ("tile_multiple_4wave_bf16", 1, 2, 128, "bf16", 2112, 64, 64, 6, 1.5, 0.0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_parity(gpu, case):
    name, B, H, d, dt, n, kh, kr, T, alpha, sink = case
    wl = Workload(name, B, H, d, dt, n, kh, kr, T, alpha, sink, seed=zlib.crc32(name.encode()) % 10000)
    run = ParityRun(wl, T)
    run.prefill()
    rep = run.decode()
    log(f"[parity] {name}: {rep}")
    assert rep.steps == T


POLICY_CASES = [
    # name, policy, B, H, d, dtype, n, k_heavy, k_recent, T
    ("averaged_bf16", "averaged", 2, 3, 128, "bf16", 300, 20, 20, 50),
    ("averaged_f32_d64", "averaged", 1, 2, 64, "f32", 129, 9, 7, 40),
    ("position_bf16", "position", 2, 2, 128, "bf16", 333, 4, 28, 40),
    ("position_f16_fill", "position", 1, 3, 64, "f16", 10, 4, 12, 30),
    ("heavy_only_bf16", "accumulated", 2, 3, 128, "bf16", 300, 32, 0, 50),
    ("heavy_only_averaged_f16", "averaged", 1, 2, 128, "f16", 200, 24, 0, 40),
    ("heavy_only_fill_f32", "accumulated", 1, 2, 64, "f32", 5, 12, 0, 30),
]


@pytest.mark.parametrize("case", POLICY_CASES, ids=[c[0] for c in POLICY_CASES])
def test_policy_parity(gpu, case):
    name, policy, B, H, d, dt, n, kh, kr, T = case
    wl = Workload(name, B, H, d, dt, n, kh, kr, T, 1.5, 0.0, seed=zlib.crc32(name.encode()) % 10000)
    run = ParityRun(wl, T, policy=policy)
    run.prefill()
    rep = run.decode()
    log(f"[parity] {name} ({policy}): {rep}")
    assert rep.steps == T


def test_policy_full_size_sampled(gpu):
    """The averaged and heavy-only variants at the OPT-6.7B layer shape (same grid as the bench)."""
    for policy, kh, kr in (("averaged", 128, 128), ("accumulated", 256, 0)):
        wl = WORKLOADS["opt6.7b_layer"].with_(k_heavy=kh, k_recent=kr)
        run = ParityRun(wl, 48, sample=sample_heads(wl, 16), policy=policy,
                        label=f"opt6.7b_layer {policy} kh={kh} kr={kr} 16 heads x 48 steps")
        run.prefill()
        rep = run.decode()
        log(f"[parity] opt6.7b_layer {policy} k_heavy={kh} k_recent={kr}: {rep}")


def test_tiny_f32_workload_full(gpu):
    wl = WORKLOADS["tiny_f32"]
    run = ParityRun(wl, wl.steps)
    run.prefill()
    rep = run.decode()
    log(f"[parity] tiny_f32: {rep}")
    assert rep.evictions_checked == wl.n_heads_total * wl.steps


def test_max_slots(gpu):
    wl = Workload("max_slots", 1, 1, 128, "bf16", 8300, 4096, 4096, 6, 1.5, 0.0, 31)
    run = ParityRun(wl, wl.steps)
    run.prefill()
    rep = run.decode()
    log(f"[parity] max_slots: {rep}")


def test_max_slots_wave_kernel(gpu):
    """1024 heads of 8192 slots, the largest cache, through the
    one-wave-per-head kernel (its 8192 logits take 32 KiB of a workgroup's
    LDS); 4 sampled heads over 4 steps, every step with a full cache."""
    wl = Workload("max_slots_1024", 8, 128, 128, "bf16", 8300, 4096, 4096, 4, 1.5, 0.0, 33)
    run = ParityRun(wl, wl.steps, sample=sample_heads(wl, 4))
    run.prefill()
    rep = run.decode()
    log(f"[parity] max slots, 1024 heads: {rep}")
    assert rep.steps == wl.steps


def test_wave_kernel_beyond_prefetch(gpu):
    """1024 heads (the one-wave-per-head kernel) with 640 slots: scores and
    positions past the 512 prefetched per head are read in the epilogue."""
    wl = Workload("wave_640", 32, 32, 128, "bf16", 900, 320, 320, 12, 1.5, 0.0, 77)
    run = ParityRun(wl, wl.steps, sample=sample_heads(wl, 12))
    run.prefill()
    rep = run.decode()
    log(f"[parity] wave kernel, 640 slots: {rep}")
    assert rep.steps == wl.steps


# Full-size workloads at the benchmark's grid, over every decode step: every
# head of the OPT-6.7B and OPT-30B layers, and a seeded sample of 512 of the
# large-batch layer's 8192 heads (whose every head is checked over the first
# four steps below).
EVERY_STEP = [("opt6.7b_layer", None), ("opt30b_layer", None), ("large_batch_f16", 512)]


@pytest.mark.parametrize("name,nsample", EVERY_STEP, ids=[f[0] for f in EVERY_STEP])
def test_full_size_every_step(gpu, name, nsample):
    wl = WORKLOADS[name]
    sample = None if nsample is None else sample_heads(wl, nsample)
    heads = wl.n_heads_total if sample is None else nsample
    run = ParityRun(wl, wl.steps, sample=sample, label=f"{name} {heads} heads x all steps")
    run.prefill()
    rep = run.decode()
    log(f"[parity] {name} full size, every step: {rep}")
    assert rep.steps == wl.steps


def test_large_batch_all_heads_first_steps(gpu):
    wl = WORKLOADS["large_batch_f16"]
    run = ParityRun(wl, 4, label="large_batch_f16 all heads x 4 steps")
    run.prefill()
    rep = run.decode()
    log(f"[parity] large_batch_f16 full size, all heads: {rep}")
    assert rep.heads == wl.n_heads_total and rep.steps == 4


def test_long_context_every_step_fused_and_split(gpu):
    """The long-context layer (256 heads x 2048 slots, prompt 16384): every
    head over all 256 steps with the fused step, then again with the split
    step (the library's chunking), both from the same oracle prefill."""
    wl = WORKLOADS["long_context"]
    fused = ParityRun(wl, wl.steps, label="long_context all heads x all steps")
    fused.prefill()
    state = fused.prefill_state
    rep = fused.decode()
    log(f"[parity] long_context fused, every step: {rep}")
    del fused
    split = ParityRun(wl, wl.steps, split_rows=0, label="long_context all heads x all steps")
    split.prefill(reuse=state)
    rep_s = split.decode()
    log(f"[parity] long_context split, every step: {rep_s}")
    assert rep.steps == rep_s.steps == wl.steps and rep.heads == wl.n_heads_total


def test_uniform_attention_closed_form_full_shape(gpu):
    """All-zero queries at the OPT-6.7B layer shape: column sums are harmonic
    differences, selection is first k_heavy + window, every step evicts
    t - k_recent and outputs are plain means of the cached values."""
    wl = WORKLOADS["opt6.7b_layer"]
    B, H, d, n, kh, kr = wl.batch, wl.heads, wl.head_dim, wl.prompt_len, wl.k_heavy, wl.k_recent
    T = 24
    dev = torch.device("cuda")
    _, K, V = make_prompt(wl)
    _, kd, vd = make_decode(wl, steps=T)
    from kv_cache_eviction_decode_amd import H2OCache
    cache = H2OCache(B, H, d, kh, kr, torch.bfloat16, wl.scale, dev)
    Qz = torch.zeros(B, H, n, d, dtype=torch.bfloat16, device=dev)
    Kg = to_device(K, "bf16", dev).view(B, H, n, d)
    Vg = to_device(V, "bf16", dev).view(B, H, n, d)
    colsum = torch.empty(B, H, n, dtype=torch.float32, device=dev)
    cache.prefill_select(Qz, Kg, Vg, colsum_out=colsum)
    Hn = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1))])
    np.testing.assert_allclose(colsum.cpu().numpy().reshape(-1, n), np.broadcast_to(Hn[n] - Hn[:n], (B * H, n)),
                               rtol=1e-4)
    expect = np.array(list(range(kh)) + list(range(n - kr, n)), dtype=np.int32)
    assert (cache.pos.cpu().numpy().reshape(-1, wl.k) == expect).all()
    allv = np.concatenate([V, vd], axis=1)  # [G, n+T, d] float64-exact values
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
        err = np.abs(out.cpu().numpy().reshape(B * H, d) - mean).max()
        assert err <= 1e-5, f"step {t}: {err}"
        members[members == pos_t - kr] = pos_t


def test_deterministic_and_resumable(gpu):
    """Two runs are bit-identical; snapshot + restore into a fresh cache and
    continue gives the same bits as the uninterrupted run."""
    from kv_cache_eviction_decode_amd import H2OCache
    wl = Workload("det", 4, 8, 128, "bf16", 700, 64, 64, 40, 1.5, 0.0, 5)
    B, H, d, n = wl.batch, wl.heads, wl.head_dim, wl.prompt_len
    dev = torch.device("cuda")
    Q, K, V = (to_device(x, "bf16", dev).view(B, H, n, d) for x in make_prompt(wl))
    qd, kd, vd = (to_device(x.transpose(1, 0, 2), "bf16", dev).view(wl.steps, B, H, d) for x in make_decode(wl))

    def run(split=None):
        c = H2OCache(B, H, d, wl.k_heavy, wl.k_recent, torch.bfloat16, wl.scale, dev)
        c.prefill_select(Q, K, V)
        outs, evs = [], []
        for t in range(wl.steps):
            if split is not None and t == split:
                st, pos_h, score_h = c.state(copy=True)
                K_snap, V_snap = c.K.clone(), c.V.clone()
                c = H2OCache(B, H, d, wl.k_heavy, wl.k_recent, torch.bfloat16, wl.scale, dev)
                c.K.copy_(K_snap)
                c.V.copy_(V_snap)
                c.pos.copy_(pos_h.to(dev))
                c.score.copy_(score_h.to(dev))
                c.restore(st.t_next, st.steps)
            o, e = c.decode_step(qd[t], kd[t], vd[t])
            outs.append(o.clone())
            evs.append(e.clone())
        return torch.stack(outs), torch.stack(evs), c.score.clone(), c.pos.clone(), c.K.clone()

    a = run()
    b = run()
    c = run(split=wl.steps // 2)
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y)
        assert torch.equal(x, z)


def test_fullcache_comparator_matches_oracle(gpu):
    from oracle import H2OOracle
    from kv_cache_eviction_decode_amd import h2o_fullcache_decode
    wl = Workload("full", 2, 4, 128, "f16", 333, 0, 1, 1, 1.5, 0.0, 8)
    B, H, d, L = wl.batch, wl.heads, wl.head_dim, wl.prompt_len
    dev = torch.device("cuda")
    Q, K, V = make_prompt(wl)
    q, _, _ = make_decode(wl, steps=1)
    out = torch.empty(B, H, d, dtype=torch.float32, device=dev)
    h2o_fullcache_decode(to_device(q[:, 0], "f16", dev).view(B, H, d), to_device(K, "f16", dev).view(B, H, L, d),
                         to_device(V, "f16", dev).view(B, H, L, d), out, wl.scale)
    # oracle: a never-full cache holding the first L-1 tokens; token L-1 arrives as the new one
    orc = H2OOracle(B * H, d, L, 1, wl.scale)
    orc.prefill(Q[:, :L - 1], K[:, :L - 1], V[:, :L - 1])
    st = orc.decode_step(q[:, 0], K[:, L - 1], V[:, L - 1])
    err = np.abs(out.cpu().numpy().reshape(B * H, d) - st.out).max()
    assert err <= out_tolerance("f16"), err


def test_state_errors_on_gpu(gpu):
    from kv_cache_eviction_decode_amd import H2OCache, H2OError, binding
    dev = torch.device("cuda")
    c = H2OCache(1, 2, 64, 4, 4, torch.bfloat16, None, dev)
    Q = torch.zeros(1, 2, 10, 64, dtype=torch.bfloat16, device=dev)
    small = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(H2OError, match="EWORKSPACE"):
        binding.h2o_prefill_select(c.desc, Q, Q, Q, small, None, None, c.device)
    c.prefill_select(Q, Q, Q)
    with pytest.raises(H2OError, match="ESTATE"):
        c.prefill_select(Q, Q, Q)
    with pytest.raises(ValueError):
        c.decode_step(torch.zeros(1, 2, 128, dtype=torch.bfloat16, device=dev), Q[:, :, 0], Q[:, :, 0])
    st = c.state()
    assert (st.n_used, st.t_next, st.k) == (8, 10, 8)
    torch.cuda.synchronize()


@pytest.mark.parametrize("policy,kh,kr", [("accumulated", 0, 256), ("position", 4, 252)],
                         ids=["window_only", "sinks_and_window"])
def test_window_policies_are_textbook_attention(gpu, policy, kh, kr):
    """With no heavy hitters (k_heavy = 0), or with the position policy (the
    first k_heavy tokens kept as sinks), the cache at step t holds exactly the
    sinks and positions t - k_recent .. t - 1, so the output is plain softmax
    attention over those plus the new token (taken before the eviction), and
    every full step evicts t - k_recent. Checked with the workload's own queries at the OPT-6.7B
    shape against attention computed directly in float64 on sampled heads."""
    wl = WORKLOADS["opt6.7b_layer"].with_(k_heavy=kh, k_recent=kr)
    B, H, d, n = wl.batch, wl.heads, wl.head_dim, wl.prompt_len
    T = 12
    dev = torch.device("cuda")
    from kv_cache_eviction_decode_amd import H2OCache
    Q, K, V = make_prompt(wl)
    qd, kd, vd = make_decode(wl, steps=T)
    cache = H2OCache(B, H, d, kh, kr, torch.bfloat16, wl.scale, dev, policy=policy)
    cache.prefill_select(*(to_device(x, "bf16", dev).view(B, H, n, d) for x in (Q, K, V)))
    expect = np.array(list(range(kh)) + list(range(n - kr, n)), dtype=np.int32)
    assert (cache.pos.cpu().numpy().reshape(-1, wl.k) == expect).all()
    sample = sample_heads(wl, 8)
    allk = np.concatenate([K[sample], kd[sample]], axis=1).astype(np.float64)
    allv = np.concatenate([V[sample], vd[sample]], axis=1).astype(np.float64)
    stage = lambda a: to_device(a.transpose(1, 0, 2), "bf16", dev).view(T, B, H, d)
    qg, kg, vg = stage(qd), stage(kd), stage(vd)
    for t in range(T):
        out, ev = cache.decode_step(qg[t], kg[t], vg[t])
        pos_t = n + t
        assert (ev.cpu().numpy() == pos_t - kr).all(), f"step {t}"
        # attention runs before the eviction: the window token about to leave still counts
        keep = np.array(list(range(kh)) + list(range(pos_t - kr, pos_t + 1)))
        gout = out.cpu().numpy().reshape(-1, d)[sample]
        for j, g in enumerate(sample):
            s = wl.scale * allk[j, keep] @ qd[g, t].astype(np.float64)
            p = np.exp(s - s.max())
            ref = (p / p.sum()) @ allv[j, keep]
            err = float(np.abs(gout[j] - ref).max())
            # inputs are the exact bf16 values on both sides: only fp32 sums and exp2 differ
            assert err <= 1e-4, f"step {t} head {g}: {err:.3g}"
    log(f"[parity] {policy} kh={kh} kr={kr}: textbook attention over {T} steps")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_never_full_cache_is_causal_attention(gpu, dtype):
    """k >= n + T: nothing is ever evicted, so each decode output is causal
    attention over the whole sequence so far and the final scores are the
    column sums of the full causal attention matrix (prompt and decode rows),
    computed here directly in float64 from the same 16-bit inputs."""
    wl = Workload("never_full", 2, 8, 128, dtype, 300, 256, 256, 20, 1.5, 0.0, 47)
    B, H, d, n, T = wl.batch, wl.heads, wl.head_dim, wl.prompt_len, wl.steps
    G, N = B * H, n + T
    dev = torch.device("cuda")
    from kv_cache_eviction_decode_amd import H2OCache
    Q, K, V = make_prompt(wl)
    qd, kd, vd = make_decode(wl)
    cache = H2OCache(B, H, d, wl.k_heavy, wl.k_recent, TORCH_DTYPE[dtype], wl.scale, dev)
    cache.prefill_select(*(to_device(x, dtype, dev).view(B, H, n, d) for x in (Q, K, V)))
    stage = lambda a: to_device(a.transpose(1, 0, 2), dtype, dev).view(T, B, H, d)
    qg, kg, vg = stage(qd), stage(kd), stage(vd)
    allq = np.concatenate([Q, qd], axis=1).astype(np.float64)
    allk = np.concatenate([K, kd], axis=1).astype(np.float64)
    allv = np.concatenate([V, vd], axis=1).astype(np.float64)
    S = wl.scale * np.einsum("gid,gjd->gij", allq, allk)
    S = np.where(np.tril(np.ones((N, N), dtype=bool)), S, -np.inf)
    P = np.exp(S - S.max(axis=2, keepdims=True))
    P /= P.sum(axis=2, keepdims=True)
    for t in range(T):
        out, ev = cache.decode_step(qg[t], kg[t], vg[t])
        assert (ev.cpu().numpy() == -1).all()
        ref = np.einsum("gj,gjd->gd", P[:, n + t], allv)
        err = float(np.abs(out.cpu().numpy().reshape(G, d) - ref).max())
        assert err <= 1e-4, f"step {t}: {err:.3g}"
    assert cache.n_used == N
    pos = cache.pos.cpu().numpy().reshape(G, -1)
    assert (pos[:, :N] == np.arange(N)).all() and (pos[:, N:] == -1).all()
    score = cache.score.cpu().numpy().reshape(G, -1)[:, :N]
    np.testing.assert_allclose(score, P.sum(axis=1), rtol=1e-4)
    log(f"[parity] never-full {dtype}: causal attention and column sums over {N} positions")


def test_reinitialised_cache_equals_fresh(gpu):
    """A cache re-initialised after a prefill and some decode steps of one
    prompt, then run on another, gives bit for bit what a fresh cache gives."""
    from kv_cache_eviction_decode_amd import H2OCache
    dev = torch.device("cuda")
    a = Workload("reinit_a", 2, 4, 128, "bf16", 400, 40, 40, 30, 1.5, 0.0, 61)
    b = a.with_(name="reinit_b", prompt_len=333, seed=62)
    B, H, d = a.batch, a.heads, a.head_dim

    def inputs(wl):
        Q, K, V = make_prompt(wl)
        qd, kd, vd = make_decode(wl)
        n = wl.prompt_len
        P = [to_device(x, "bf16", dev).view(B, H, n, d) for x in (Q, K, V)]
        D = [to_device(x.transpose(1, 0, 2), "bf16", dev).view(wl.steps, B, H, d) for x in (qd, kd, vd)]
        return P, D

    def run(cache, wl, steps):
        P, D = inputs(wl)
        cache.prefill_select(*P)
        outs = []
        for t in range(steps):
            out, ev = cache.decode_step(D[0][t], D[1][t], D[2][t])
            outs.append((out.clone(), ev.clone()))
        torch.cuda.synchronize()
        return outs

    used = H2OCache(B, H, d, a.k_heavy, a.k_recent, torch.bfloat16, a.scale, dev)
    run(used, a, 17)
    from kv_cache_eviction_decode_amd.binding import h2o_cache_init
    h2o_cache_init(used.desc, B, H, d, a.k_heavy, a.k_recent, "accumulated", a.scale,
                   used.K, used.V, used.score, used.pos, None)
    got = run(used, b, b.steps)
    fresh = H2OCache(B, H, d, a.k_heavy, a.k_recent, torch.bfloat16, a.scale, dev)
    want = run(fresh, b, b.steps)
    for t, ((go, ge), (wo, we)) in enumerate(zip(got, want)):
        assert torch.equal(go, wo) and torch.equal(ge, we), f"step {t}"
    for x, y in ((used.K, fresh.K), (used.V, fresh.V), (used.score, fresh.score), (used.pos, fresh.pos)):
        assert torch.equal(x, y)
    log("[parity] re-initialised cache equals a fresh one")


def test_two_caches_on_two_streams(gpu):
    """Two caches decoded concurrently on two streams (default priority) give
    bit for bit what the same calls give one after the other on one stream:
    the library keeps no state shared between calls."""
    from kv_cache_eviction_decode_amd import H2OCache
    dev = torch.device("cuda")
    wls = [Workload("streams_a", 4, 8, 128, "bf16", 500, 64, 64, 24, 1.5, 0.0, 71),
           Workload("streams_b", 4, 8, 128, "bf16", 700, 64, 64, 24, 1.2, 0.0, 72)]
    data = []
    for wl in wls:
        Q, K, V = make_prompt(wl)
        qd, kd, vd = make_decode(wl)
        B, H, n, d = wl.batch, wl.heads, wl.prompt_len, wl.head_dim
        data.append(([to_device(x, "bf16", dev).view(B, H, n, d) for x in (Q, K, V)],
                     [to_device(x.transpose(1, 0, 2), "bf16", dev).view(wl.steps, B, H, d) for x in (qd, kd, vd)]))

    def run(streams):
        caches = [H2OCache(wl.batch, wl.heads, wl.head_dim, wl.k_heavy, wl.k_recent, torch.bfloat16, wl.scale, dev)
                  for wl in wls]
        outs = [torch.empty(wls[0].steps, wl.batch, wl.heads, wl.head_dim, device=dev) for wl in wls]
        evs = [torch.empty(wls[0].steps, wl.batch, wl.heads, dtype=torch.int32, device=dev) for wl in wls]
        torch.cuda.synchronize()
        for i, (c, (P, D)) in enumerate(zip(caches, data)):
            with torch.cuda.stream(streams[i]):
                c.prefill_select(*P, stream=streams[i])
        for t in range(wls[0].steps):
            for i, (c, (P, D)) in enumerate(zip(caches, data)):
                with torch.cuda.stream(streams[i]):
                    c.decode_step(D[0][t], D[1][t], D[2][t], outs[i][t], evs[i][t], stream=streams[i])
        torch.cuda.synchronize()
        return outs, evs, caches

    s0 = torch.cuda.current_stream()
    seq = run([s0, s0])
    par = run([torch.cuda.Stream(), torch.cuda.Stream()])
    for i in range(2):
        assert torch.equal(seq[0][i], par[0][i]) and torch.equal(seq[1][i], par[1][i])
        for x, y in ((seq[2][i].score, par[2][i].score), (seq[2][i].pos, par[2][i].pos), (seq[2][i].K, par[2][i].K)):
            assert torch.equal(x, y)
    log("[parity] two caches on two streams match one stream")


def test_maximum_prompt_closed_form(gpu):
    """One head at the largest prompt the library accepts (H2O_MAX_PROMPT), with
    all-zero queries: the column sums are the harmonic differences H_n - H_j
    at every position, the selection is the first k_heavy plus the window, and
    decode evicts t - k_recent. Exercises every prefill tile and the largest
    row offsets the kernels address."""
    from kv_cache_eviction_decode_amd import H2OCache
    from kv_cache_eviction_decode_amd.binding import H2O_MAX_PROMPT
    n = H2O_MAX_PROMPT
    wl = Workload("max_prompt", 1, 1, 128, "bf16", n, 1024, 1024, 4, 1.5, 0.0, 83)
    d, kh, kr = wl.head_dim, wl.k_heavy, wl.k_recent
    dev = torch.device("cuda")
    _, K, V = make_prompt(wl)
    _, kd, vd = make_decode(wl)
    cache = H2OCache(1, 1, d, kh, kr, torch.bfloat16, wl.scale, dev)
    colsum = torch.empty(1, 1, n, dtype=torch.float32, device=dev)
    log(f"[parity] max prompt: prefill of {n} tokens")
    cache.prefill_select(torch.zeros(1, 1, n, d, dtype=torch.bfloat16, device=dev),
                         to_device(K, "bf16", dev).view(1, 1, n, d), to_device(V, "bf16", dev).view(1, 1, n, d),
                         colsum_out=colsum)
    del K, V
    Hn = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1, dtype=np.float64))])
    np.testing.assert_allclose(colsum.view(-1).cpu().numpy(), Hn[n] - Hn[:n], rtol=1e-4)
    expect = np.array(list(range(kh)) + list(range(n - kr, n)), dtype=np.int32)
    assert (cache.pos.view(-1).cpu().numpy() == expect).all()
    qz = torch.zeros(1, 1, d, dtype=torch.bfloat16, device=dev)
    for t in range(wl.steps):
        _, ev = cache.decode_step(qz, to_device(kd[:, t], "bf16", dev).view(1, 1, d),
                                  to_device(vd[:, t], "bf16", dev).view(1, 1, d))
        assert int(ev.item()) == n + t - kr, f"step {t}"
    log("[parity] max prompt: closed form holds")
