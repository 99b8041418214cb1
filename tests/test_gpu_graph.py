"""Decode steps captured in a HIP graph and replayed.

A decode step launches only library kernels on the caller's stream (no
device-wide synchronisation, no host read-back, no memset), so a sequence of
steps can be captured once and replayed as one graph, the way a serving loop
removes launch overhead. The descriptor's host counters advance while the
steps are captured; the graph holds the positions of the captured steps, so
every replay starts from the same device state. Each replay is checked
against eager execution from that state, with eager work and
synchronisations between the replays.
"""
import numpy as np
import pytest
import torch

from kv_cache_eviction_decode_amd import H2OCache
from workload import Workload, make_decode, make_prompt

pytestmark = pytest.mark.gpu

T = 12


def _inputs(wl, dev):
    Q, K, V = make_prompt(wl)
    qd, kd, vd = make_decode(wl, steps=T)
    B, H, n, d = wl.batch, wl.heads, wl.prompt_len, wl.head_dim
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)
    P = [up(x).view(B, H, n, d) for x in (Q, K, V)]
    D = [up(x.transpose(1, 0, 2)).view(T, B, H, d) for x in (qd, kd, vd)]
    return P, D


def _state(c):
    st = [c.K, c.V, c.score, c.pos] + ([c.v_qparam] if c.quant else [])
    return [x.clone() for x in st]


def _load(c, snap):
    for dst, src in zip([c.K, c.V, c.score, c.pos] + ([c.v_qparam] if c.quant else []), snap):
        dst.copy_(src)


@pytest.mark.parametrize("mode", ["fused", "split", "u8", "u4", "u2"])
def test_decode_steps_replay_from_a_graph(gpu, mode):
    wl = Workload("graph_" + mode, 2, 4, 128, "bf16", 300, 24, 24, T, 1.5, 0.0, seed=55)
    dev = torch.device("cuda")
    P, D = _inputs(wl, dev)
    B, H, d = wl.batch, wl.heads, wl.head_dim
    c = H2OCache(B, H, d, wl.k_heavy, wl.k_recent, torch.bfloat16, wl.scale, dev,
                 quant=mode if mode in ("u8", "u4", "u2") else None)
    c.prefill_select(*P)
    outs = torch.empty(T, B, H, d, dtype=torch.float32, device=dev)
    evs = torch.empty(T, B, H, dtype=torch.int32, device=dev)
    step = (lambda t: c.decode_step_split(D[0][t], D[1][t], D[2][t], outs[t], evs[t])) if mode == "split" else \
        (lambda t: c.decode_step(D[0][t], D[1][t], D[2][t], outs[t], evs[t]))
    if mode == "split":
        c.split_workspace()  # allocated before capture
    torch.cuda.synchronize()
    snap, t0 = _state(c), c.t_next

    # eager reference from the snapshot
    for t in range(T):
        step(t)
    torch.cuda.synchronize()
    ref_out, ref_ev, ref_state = outs.clone(), evs.clone(), _state(c)

    # capture the same T steps
    _load(c, snap)
    c.restore(t0)
    outs.zero_()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for t in range(T):
                step(t)
    torch.cuda.synchronize()
    assert c.t_next == t0 + T

    for rep in range(3):
        _load(c, snap)
        outs.fill_(float("nan"))
        evs.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs, ref_out), f"replay {rep}: outputs differ"
        assert torch.equal(evs, ref_ev), f"replay {rep}: evictions differ"
        for a, b in zip(_state(c), ref_state):
            assert torch.equal(a, b), f"replay {rep}: cache state differs"
        # eager work between replays
        _ = (outs * 2).sum().item()


@pytest.mark.parametrize("mode", ["select", "attention", "u4"])
def test_init_and_prefill_replay_from_a_graph(gpu, mode):
    """Cache initialisation and prefill (clear kernel, scoring passes,
    selection and gather; for "attention" also the prompt's output) captured
    once and replayed three times, with eager work between the replays: every
    replay reproduces the eager result bit for bit."""
    from kv_cache_eviction_decode_amd.binding import h2o_cache_init, h2o_cache_init_quant
    wl = Workload("graph_prefill_" + mode, 2, 4, 128, "bf16", 700, 40, 40, T, 1.5, 0.0, seed=57)
    dev = torch.device("cuda")
    P, _ = _inputs(wl, dev)
    B, H, d, n = wl.batch, wl.heads, wl.head_dim, wl.prompt_len
    quant = "u4" if mode == "u4" else None
    c = H2OCache(B, H, d, wl.k_heavy, wl.k_recent, torch.bfloat16, wl.scale, dev, quant=quant)
    c.workspace(n)
    colsum = torch.empty(B, H, n, dtype=torch.float32, device=dev)
    pout = torch.empty(B, H, n, d, dtype=torch.float32, device=dev)

    def step(stream=None):
        if quant:
            h2o_cache_init_quant(c.desc, B, H, d, wl.k_heavy, wl.k_recent, "accumulated", torch.bfloat16, wl.scale,
                                 quant, c.K, c.V, c.k_qparam, c.v_qparam, c.score, c.pos, stream)
        else:
            h2o_cache_init(c.desc, B, H, d, wl.k_heavy, wl.k_recent, "accumulated", wl.scale,
                           c.K, c.V, c.score, c.pos, stream)
        if mode == "attention":
            c.prefill_attention(*P, out=pout, colsum_out=colsum, stream=stream)
        else:
            c.prefill_select(*P, colsum_out=colsum, stream=stream)

    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in _state(c) + [colsum, pout]]

    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for x in _state(c):
            x.zero_()
        colsum.fill_(float("nan"))
        if mode == "attention":
            pout.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(_state(c) + [colsum, pout], ref):
            assert torch.equal(a, b), f"replay {rep}: state differs"
        _ = (colsum * 2).sum().item()  # eager work between replays
