"""Pins of the fp64 oracle against things other than itself (CPU only).

* brute force: a position-indexed, loop-based replay (oracle/brute.py) with
  exhaustive subset search for the prefill selection, on many tiny cases;
* closed forms: with all-zero queries every attention row is uniform, so
  prefill column sums are harmonic-number differences and H2O reduces to
  "first k_heavy tokens + sliding window";
* textbook special cases: a cache that never fills is plain causal attention
  (checked against torch's scaled_dot_product_attention in float64) and
  k_heavy = 0 is sliding-window attention;
* hand-worked examples under tests/golden/;
* invariants of the method at a realistic (small) workload;
* planted mistakes: each mutant of an oracle step must fail a pin.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle.h2o_oracle as oh
from oracle import H2OOracle, brute_run
from oracle.h2o_oracle import select_prefill
from workload import Workload, make_decode, make_prompt

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- helpers
def _tiny_case(seed, n, T, d, heads=2):
    """Small random inputs with a heavy-hitter direction (as in the workload recipe)."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    s = np.minimum((1.0 - rng.random((heads, n + T))) ** (-1 / 1.5), 4.0)
    Q = rng.standard_normal((heads, n, d)) + 2 * u
    K = rng.standard_normal((heads, n, d)) + s[:, :n, None] * u
    V = rng.standard_normal((heads, n, d))
    q = rng.standard_normal((heads, T, d)) + 2 * u
    k = rng.standard_normal((heads, T, d)) + s[:, n:, None] * u
    v = rng.standard_normal((heads, T, d))
    return Q, K, V, q, k, v


def _run_oracle(Q, K, V, q, k, v, k_heavy, k_recent, scale, policy="accumulated"):
    G, n, d = Q.shape
    orc = H2OOracle(G, d, k_heavy, k_recent, scale, policy)
    pre = orc.prefill(Q, K, V)
    kept = [set(orc.pos[g][orc.pos[g] >= 0].tolist()) for g in range(G)]
    steps = [orc.decode_step(q[:, t], k[:, t], v[:, t]) for t in range(q.shape[1])]
    return orc, pre, kept, steps


def _compare_with_brute(Q, K, V, q, k, v, k_heavy, k_recent, scale, tol=1e-12, policy="accumulated"):
    orc, pre, kept, steps = _run_oracle(Q, K, V, q, k, v, k_heavy, k_recent, scale, policy)
    for g in range(Q.shape[0]):
        br = brute_run(Q[g], K[g], V[g], q[g], k[g], v[g], k_heavy, k_recent, scale, policy)
        np.testing.assert_allclose(pre.colsum[g], br["colsum"], rtol=0, atol=tol)
        assert kept[g] == br["kept"]
        for t, st in enumerate(steps):
            assert st.evicted[g] == br["evicted"][t], (g, t)
            np.testing.assert_allclose(st.out[g], br["outs"][t], rtol=0, atol=tol)
        live = orc.pos[g] >= 0
        assert set(orc.pos[g][live].tolist()) == br["alive"]
        for p_, s_ in zip(orc.pos[g][live], orc.score[g][live]):
            assert abs(s_ - br["acc"][p_]) <= tol


# ----------------------------------------------------------------------------- brute force
TINY = [
    # (n, T, d, k_heavy, k_recent)
    (0, 6, 4, 1, 1), (1, 5, 4, 2, 1), (3, 8, 4, 2, 2), (6, 10, 8, 2, 1),
    (9, 10, 8, 3, 2), (12, 8, 4, 4, 2), (12, 10, 8, 0, 3), (10, 9, 4, 1, 4),
    (7, 10, 8, 3, 3), (11, 6, 4, 5, 1), (5, 0, 4, 1, 1), (8, 10, 4, 6, 1),
]


@pytest.mark.parametrize("case", TINY)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_oracle_matches_brute_force(case, seed):
    n, T, d, kh, kr = case
    data = _tiny_case(100 * seed + n, n, T, d)
    _compare_with_brute(*data, kh, kr, 1 / math.sqrt(d))


# ----------------------------------------------------------------------------- closed form q = 0
def test_uniform_attention_closed_form():
    """All-zero queries: P[i, j] = 1/(i+1), so c_j = H_n - H_j, and H2O keeps
    the first k_heavy tokens plus the window; the victim is always t - k_recent."""
    G, n, d, kh, kr, T = 3, 200, 16, 20, 20, 60
    rng = np.random.default_rng(5)
    K = rng.standard_normal((G, n, d))
    V = rng.standard_normal((G, n, d))
    kd = rng.standard_normal((G, T, d))
    vd = rng.standard_normal((G, T, d))
    Q = np.zeros((G, n, d))
    qd = np.zeros((G, T, d))
    orc = H2OOracle(G, d, kh, kr, 0.125)
    pre = orc.prefill(Q, K, V)
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1))])
    np.testing.assert_allclose(pre.colsum, np.broadcast_to(H[n] - H[:n], (G, n)), rtol=1e-13)
    expect = list(range(kh)) + list(range(n - kr, n))
    assert all(orc.pos[g].tolist() == expect for g in range(G))
    allv = np.concatenate([V, vd], axis=1)
    for t in range(T):
        members = [orc.pos[g][orc.pos[g] >= 0] for g in range(G)]
        st = orc.decode_step(qd[:, t], kd[:, t], vd[:, t])
        np.testing.assert_allclose(st.probs, 1.0 / (orc.k + 1), rtol=1e-14)
        for g in range(G):
            mean = allv[g][np.concatenate([members[g], [n + t]])].mean(axis=0)
            np.testing.assert_allclose(st.out[g], mean, rtol=0, atol=1e-13)
        assert (st.evicted == n + t - kr).all()


def test_uniform_attention_fills_then_streams():
    """Prompt shorter than the cache: no eviction until full; then the token
    leaving the window goes (its score is the smallest eligible one)."""
    G, n, d, kh, kr, T = 2, 5, 8, 4, 3, 12
    rng = np.random.default_rng(9)
    orc = H2OOracle(G, d, kh, kr, 0.3)
    orc.prefill(np.zeros((G, n, d)), rng.standard_normal((G, n, d)), rng.standard_normal((G, n, d)))
    ev = []
    for t in range(T):
        st = orc.decode_step(np.zeros((G, d)), rng.standard_normal((G, d)), rng.standard_normal((G, d)))
        assert orc.n_used == min(orc.k, n + t + 1)
        ev.append(int(st.evicted[0]))
    k = kh + kr
    assert ev == [-1] * (k - n) + [n + t - kr for t in range(k - n, T)]


# ----------------------------------------------------------------------------- golden fixtures
def _load_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (x.strip() for x in line.split("=", 1))
            vals[key] = val
    return vals


def _fracs(s):
    return [float(Fraction(x)) for x in s.split()]


def _golden_inputs(g):
    n, d, steps = int(g["n"]), int(g["d"]), int(g["steps"])
    N = n + steps
    if g.get("query") == "zero":
        qs = np.zeros((N, d))
        keys = np.ones((N, d))
        scale = 1 / math.sqrt(d)
    else:
        qs = np.ones((N, d))
        w = [float(x) for x in (g["prompt_weights"] + " " + g["decode_weights"]).split()]
        keys = np.log(np.array(w))[:, None]
        scale = 1.0
    if g["value"] == "position_and_one":
        vals = np.stack([np.arange(N, dtype=float), np.ones(N)], axis=1)
    else:
        vals = np.arange(N, dtype=float)[:, None]
    return n, steps, qs, keys, vals, scale


@pytest.mark.parametrize("name", ["illustration_budget3.txt", "weighted_budget3.txt", "averaged_budget3.txt",
                                  "heavy_only_budget2.txt"])
def test_golden_hand_worked(name):
    g = _load_golden(name)
    n, steps, qs, keys, vals, scale = _golden_inputs(g)
    d = qs.shape[1]
    orc = H2OOracle(1, d, int(g["k_heavy"]), int(g["k_recent"]), scale, g.get("policy", "accumulated"))
    pre = orc.prefill(qs[None, :n], keys[None, :n], vals[None, :n])
    np.testing.assert_allclose(pre.colsum[0], _fracs(g["colsum"]), rtol=1e-13)
    assert orc.pos[0].tolist() == [int(x) for x in g["after_prefill_pos"].split()]
    np.testing.assert_allclose(orc.score[0], _fracs(g["after_prefill_score"]), rtol=1e-13)
    for t in range(steps):
        st = orc.decode_step(qs[None, n + t], keys[None, n + t], vals[None, n + t])
        assert int(st.evicted[0]) == int(g[f"step{t}_evicted"])
        np.testing.assert_allclose(st.out[0], _fracs(g[f"step{t}_out"]), rtol=1e-13)
    assert orc.pos[0].tolist() == [int(x) for x in g["final_pos"].split()]
    np.testing.assert_allclose(orc.score[0], _fracs(g["final_score"]), rtol=1e-13)


def test_averaged_fixture_discriminates():
    """On the averaged fixture's inputs accumulated attention keeps position 0
    at prefill and evicts 4 at the third step, so the fixture pins the averaging."""
    g = _load_golden("averaged_budget3.txt")
    n, steps, qs, keys, vals, scale = _golden_inputs(g)
    orc = H2OOracle(1, 1, int(g["k_heavy"]), int(g["k_recent"]), scale, "accumulated")
    orc.prefill(qs[None, :n], keys[None, :n], vals[None, :n])
    assert orc.pos[0].tolist() == [0, 2, 3]
    ev = [int(orc.decode_step(qs[None, n + t], keys[None, n + t], vals[None, n + t]).evicted[0])
          for t in range(steps)]
    assert ev[2] == 4


# ----------------------------------------------------------------------------- textbook special cases
def _sdpa(q, k, v, scale, mask=None, causal=False):
    import torch
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))[None]
    out = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=None if mask is None else torch.from_numpy(mask)[None],
        is_causal=causal, scale=scale)
    return out[0].numpy()


def test_never_full_cache_is_causal_attention():
    """k >= n + T: no eviction ever; outputs are causal attention over the whole
    sequence and final scores are the full attention matrix's column sums."""
    import torch
    G, n, T, d = 2, 40, 25, 16
    Q, K, V, q, k, v = _tiny_case(11, n, T, d, heads=G)
    scale = 1 / math.sqrt(d)
    orc, pre, _, steps = _run_oracle(Q, K, V, q, k, v, 40, 30, scale)
    for g in range(G):
        allq = np.concatenate([Q[g], q[g]])
        allk = np.concatenate([K[g], k[g]])
        allv = np.concatenate([V[g], v[g]])
        ref = _sdpa(allq, allk, allv, scale, causal=True)
        got = np.stack([st.out[g] for st in steps])
        np.testing.assert_allclose(got, ref[n:], rtol=0, atol=1e-12)
        S = torch.from_numpy(scale * allq @ allk.T)
        S = S.masked_fill(~torch.ones(n + T, n + T, dtype=torch.bool).tril(), float("-inf"))
        P = torch.softmax(S, dim=1).numpy()
        np.testing.assert_allclose(pre.colsum[g], P[:n, :n].sum(0), rtol=0, atol=1e-12)
        np.testing.assert_allclose(orc.score[g][:n + T], P.sum(0), rtol=0, atol=1e-12)
        assert orc.pos[g][:n + T].tolist() == list(range(n + T))
        assert all(st.evicted[g] == -1 for st in steps)


def test_local_only_is_sliding_window_attention():
    """k_heavy = 0: query t attends exactly to positions t - k_recent .. t."""
    G, n, T, d, w = 2, 30, 40, 8, 6
    Q, K, V, q, k, v = _tiny_case(12, n, T, d, heads=G)
    scale = 1 / math.sqrt(d)
    orc, _, kept, steps = _run_oracle(Q, K, V, q, k, v, 0, w, scale)
    i = np.arange(n + T)
    band = (i[None, :] <= i[:, None]) & (i[None, :] >= i[:, None] - w)
    for g in range(G):
        assert kept[g] == set(range(n - w, n))
        ref = _sdpa(np.concatenate([Q[g], q[g]]), np.concatenate([K[g], k[g]]),
                    np.concatenate([V[g], v[g]]), scale, mask=band)
        got = np.stack([st.out[g] for st in steps])
        np.testing.assert_allclose(got, ref[n:], rtol=0, atol=1e-12)
        assert [int(st.evicted[g]) for st in steps] == [n + t - w for t in range(T)]


# ----------------------------------------------------------------------------- invariants
@pytest.mark.parametrize("prompt_len", [150, 10])
def test_invariants_on_pareto_workload(prompt_len):
    wl = Workload("inv", 1, 4, 32, "bf16", prompt_len, 12, 12, 80, 1.5, 4.0, 77)
    Q, K, V = make_prompt(wl)
    q, k, v = make_decode(wl)
    orc = H2OOracle(wl.n_heads_total, wl.head_dim, wl.k_heavy, wl.k_recent, wl.scale)
    pre = orc.prefill(Q, K, V)
    n = wl.prompt_len
    dropped = np.zeros(orc.G)
    for g in range(orc.G):
        kept = orc.pos[g][orc.pos[g] >= 0]
        dropped[g] = pre.colsum[g].sum() - pre.colsum[g][kept].sum()
    np.testing.assert_allclose(orc.score.sum(1) + dropped, n, rtol=1e-12)
    for t in range(wl.steps):
        before_pos, before_score = orc.pos.copy(), orc.score.copy()
        pos_t = orc.t
        full = orc.n_used == orc.k
        st = orc.decode_step(q[:, t], k[:, t], v[:, t])
        rows = np.arange(orc.G)
        # 1. occupancy
        assert orc.n_used == min(orc.k, n + t + 1)
        assert ((orc.pos >= 0).sum(1) == orc.n_used).all()
        # 2. recent window (pos_t - k_recent, pos_t] always cached
        for g in range(orc.G):
            window = set(range(max(0, pos_t - wl.k_recent + 1), pos_t + 1))
            assert window <= set(orc.pos[g].tolist())
        # 3. probabilities sum to one
        np.testing.assert_allclose(st.probs.sum(1), 1.0, rtol=0, atol=1e-12)
        # 4. scores of slots keeping their token never decrease
        same = (orc.pos == before_pos) & (before_pos >= 0)
        assert (orc.score[same] >= before_score[same]).all()
        # 6./7. exactly one eviction when full, of the smallest eligible score
        if full:
            assert (st.evicted >= 0).all()
            upd = before_score.copy()
            upd[:, :orc.k] += st.probs[:, :orc.k]
            victim_score = upd[rows, st.slot]
            elig = (before_pos <= pos_t - wl.k_recent)
            assert (np.where(elig, upd, np.inf).min(1) == victim_score).all()
            dropped += victim_score
        else:
            assert (st.evicted == -1).all()
        # 5. mass conservation: every attention row sums to one
        np.testing.assert_allclose(orc.score.sum(1) + dropped, n + t + 1, rtol=1e-12)


# ----------------------------------------------------------------------------- planted mistakes
def _mutant_is_caught(monkeypatch, attr, fake):
    monkeypatch.setattr(oh, attr, fake)
    caught = 0
    for case in [(9, 10, 8, 3, 2), (12, 8, 4, 4, 2), (6, 10, 8, 2, 1)]:
        n, T, d, kh, kr = case
        data = _tiny_case(3 + n, n, T, d)
        try:
            _compare_with_brute(*data, kh, kr, 1 / math.sqrt(d))
        except AssertionError:
            caught += 1
    return caught > 0


def test_planted_mistakes_are_caught(monkeypatch):
    orig_probs = oh.causal_attention_probs
    orig_rows = oh.causal_attention_probs_rows
    orig_select = oh.select_prefill

    def no_diagonal(Qb, K, s, r0):
        P = orig_rows(Qb, K, s, r0)
        P = np.where(np.arange(K.shape[0])[None, :] < np.arange(r0, r0 + Qb.shape[0])[:, None], P, 0.0)
        return P / np.maximum(P.sum(1, keepdims=True), 1e-300)

    mutants = {
        # diagonal dropped from prefill attention
        "causal_attention_probs_rows": no_diagonal,
        # row sums instead of column sums
        "prefill_column_sums": lambda Q, K, s: orig_probs(Q, K, s).sum(axis=1),
        # recent window off by one
        "eligible_slots": lambda pos, t, kr: (pos >= 0) & (pos < t - kr),
        # evict the largest value instead of the smallest
        "choose_victim": lambda value, pos, e, exact=False: (np.argmax(np.where(e, value, -np.inf), 1),
                                                             np.full(value.shape[0], np.inf)),
        # heavy hitters chosen by smallest score
        "select_prefill": lambda c, kh, kr, policy="accumulated": orig_select(-np.asarray(c) + 10, kh, kr, policy),
    }
    for attr, fake in mutants.items():
        with monkeypatch.context() as m:
            assert _mutant_is_caught(m, attr, fake), attr


# ----------------------------------------------------------------------------- policies
POLICY_CASES = [
    # (n, T, d, k_heavy, k_recent)
    (9, 10, 8, 3, 2), (12, 8, 4, 4, 2), (6, 10, 8, 2, 1), (3, 8, 4, 2, 2),
    (10, 9, 4, 3, 0), (8, 10, 8, 4, 0), (5, 8, 4, 1, 0), (0, 6, 4, 2, 0),
]


@pytest.mark.parametrize("policy", ["averaged", "position", "accumulated"])
@pytest.mark.parametrize("case", POLICY_CASES)
@pytest.mark.parametrize("seed", [0, 1])
def test_policies_match_brute_force(policy, case, seed):
    n, T, d, kh, kr = case
    data = _tiny_case(50 * seed + n + 7, n, T, d)
    _compare_with_brute(*data, kh, kr, 1 / math.sqrt(d), policy=policy)


def test_position_policy_is_sink_plus_window_attention():
    """The position policy keeps the first k_heavy tokens and the last k_recent:
    query t attends to positions < k_heavy and to t - k_recent .. t (StreamingLLM)."""
    G, n, T, d, sinks, w = 2, 30, 40, 8, 4, 6
    Q, K, V, q, k, v = _tiny_case(21, n, T, d, heads=G)
    scale = 1 / math.sqrt(d)
    orc, _, kept, steps = _run_oracle(Q, K, V, q, k, v, sinks, w, scale, "position")
    i = np.arange(n + T)
    mask = (i[None, :] <= i[:, None]) & ((i[None, :] >= i[:, None] - w) | (i[None, :] < sinks))
    for g in range(G):
        assert kept[g] == set(range(sinks)) | set(range(n - w, n))
        ref = _sdpa(np.concatenate([Q[g], q[g]]), np.concatenate([K[g], k[g]]),
                    np.concatenate([V[g], v[g]]), scale, mask=mask)
        got = np.stack([st.out[g] for st in steps])
        np.testing.assert_allclose(got, ref[n:], rtol=0, atol=1e-12)
        assert [int(st.evicted[g]) for st in steps] == [n + t - w for t in range(T)]


def test_heavy_only_uniform_attention_rejects_every_new_token():
    """k_recent = 0 with all-zero queries: older tokens always hold more
    accumulated attention, so each new token is the one evicted and the
    cache keeps the prompt's first k tokens."""
    G, n, d, k, T = 2, 20, 8, 6, 15
    rng = np.random.default_rng(4)
    orc = H2OOracle(G, d, k, 0, 0.3)
    orc.prefill(np.zeros((G, n, d)), rng.standard_normal((G, n, d)), rng.standard_normal((G, n, d)))
    assert all(orc.pos[g].tolist() == list(range(k)) for g in range(G))
    for t in range(T):
        st = orc.decode_step(np.zeros((G, d)), rng.standard_normal((G, d)), rng.standard_normal((G, d)))
        assert (st.evicted == n + t).all() and (st.slot == -1).all()
        np.testing.assert_allclose(st.probs, 1.0 / (k + 1), rtol=1e-14)
    assert all(orc.pos[g].tolist() == list(range(k)) for g in range(G))


def test_averaged_value_counts_queries():
    """Averaged policy: at the end of the prompt a token at j has been seen by
    n - j queries; with uniform attention its average is (H_n - H_j) / (n - j)."""
    n = 40
    c = np.array([sum(1.0 / (i + 1) for i in range(j, n)) for j in range(n)])
    keep, _ = select_prefill(c, 5, 5, "averaged")
    avg = c[:n - 5] / (n - np.arange(n - 5))
    expect = sorted(np.argsort(-avg, kind="stable")[:5].tolist())
    assert keep[:5].tolist() == expect


def test_prefill_attention_is_causal_sdpa():
    """The prompt's attention output and row normalisers against torch's
    scaled_dot_product_attention (float64, causal) and a log-sum-exp written
    out with torch; q = 0 gives running means of V and lse_i = log(i + 1)."""
    import torch

    from oracle.h2o_oracle import prefill_attention
    rng = np.random.default_rng(21)
    n, d, scale = 37, 16, 0.31
    Q, K, V = (rng.standard_normal((n, d)) for _ in range(3))
    O, lse = prefill_attention(Q, K, V, scale)
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (Q, K, V))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)[0, 0].numpy()
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)
    s = scale * torch.from_numpy(Q) @ torch.from_numpy(K).T
    s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=1).numpy(), rtol=0, atol=1e-12)
    O0, lse0 = prefill_attention(np.zeros((n, d)), K, V, scale)
    np.testing.assert_allclose(O0, np.cumsum(V, 0) / np.arange(1, n + 1)[:, None], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse0, np.log(np.arange(1, n + 1)), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- row blocks
@pytest.mark.parametrize("block", [1, 7, 64])
def test_row_blocked_column_sums_equal_whole_matrix(block):
    """Column sums taken over row blocks equal those of the whole causal
    attention matrix (each row's softmax is complete within its block)."""
    rng = np.random.default_rng(block)
    n, d = 150, 16
    Q, K = rng.standard_normal((n, d)) + 1.0, rng.standard_normal((n, d))
    whole = oh.causal_attention_probs(Q, K, 0.3).sum(axis=0)
    np.testing.assert_allclose(oh.prefill_column_sums(Q, K, 0.3, block=block), whole, rtol=1e-13, atol=1e-15)
    # all-zero queries: uniform rows, c_j = H_n - H_j, whatever the blocking
    Hn = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1))])
    np.testing.assert_allclose(oh.prefill_column_sums(np.zeros((n, d)), K, 0.3, block=block), Hn[n] - Hn[:n],
                               rtol=1e-13)


def test_threaded_oracle_is_bit_identical():
    rng = np.random.default_rng(5)
    G, n, d = 6, 90, 8
    Q, K, V = (rng.standard_normal((G, n, d)) for _ in range(3))
    q, k, v = (rng.standard_normal((G, 40, d)) for _ in range(3))
    a, b = H2OOracle(G, d, 10, 10, 0.35), H2OOracle(G, d, 10, 10, 0.35, workers=4)
    ra, rb = a.prefill(Q, K, V), b.prefill(Q, K, V)
    assert np.array_equal(ra.colsum, rb.colsum) and np.array_equal(a.pos, b.pos)
    assert np.array_equal(a.score, b.score) and np.array_equal(a.K, b.K)
    for t in range(40):
        sa, sb = a.decode_step(q[:, t], k[:, t], v[:, t]), b.decode_step(q[:, t], k[:, t], v[:, t])
        assert np.array_equal(sa.out, sb.out) and np.array_equal(sa.evicted, sb.evicted)
        assert np.array_equal(a.score, b.score) and np.array_equal(a.pos, b.pos)


def test_snapshot_restore_round_trip():
    rng = np.random.default_rng(9)
    G, n, d = 3, 40, 8
    Q, K, V = (rng.standard_normal((G, n, d)) for _ in range(3))
    q, k, v = (rng.standard_normal((G, 6, d)) for _ in range(3))
    a = H2OOracle(G, d, 8, 8, 0.35)
    a.prefill(Q, K, V)
    snap = a.snapshot()
    first = [a.decode_step(q[:, t], k[:, t], v[:, t]).evicted for t in range(6)]
    b = H2OOracle(G, d, 8, 8, 0.35)
    b.restore(snap)
    again = [b.decode_step(q[:, t], k[:, t], v[:, t]).evicted for t in range(6)]
    assert all(np.array_equal(x, y) for x, y in zip(first, again))
    assert np.array_equal(a.score, b.score) and np.array_equal(a.K, b.K) and a.t == b.t
