"""Brute-force replay of H2O for tiny inputs: the independent check of the fp64 oracle.

TEST INFRASTRUCTURE (same rules as the oracle: only tests may run it).

Citations ("H2O §x") refer to the page "H2O: Heavy-Hitter Oracle for Efficient
Generative Inference of Large Language Models" (paperlayer.ai summary of arXiv
2306.14048v3).

This replay deliberately uses a different formulation from the oracle, so that
a mistake in one does not repeat in the other:

* it is indexed by token position, not by cache slot: it keeps every token's
  key and value and a set of alive positions;
* attention weights use the raw definition exp(s) / sum exp(s), with plain
  Python loops and ``math.exp`` (no max shift, no numpy);
* the accumulated score of a token is the sum of the attention every query
  gave it while it was alive (H2O §1, §4.1);
* the prefill selection enumerates every subset of k_heavy candidates and
  keeps the one with the largest total accumulated attention (the greedy
  top-k of H2O §3.2 and §D is optimal for this additive objective, so the
  exhaustive search pins it);
* the eviction is the set-function form of H2O §D "Cache eviction": among the
  positions that may leave, remove the one whose removal leaves the cache
  with the largest total value.

Values per policy (see the oracle): accumulated score; averaged score (the
accumulated score over the count of queries that attended to the token,
counted here by an explicit per-position counter rather than a formula); or
minus the position (StreamingLLM's sinks plus window). With no recent window
(k_recent = 0) the new token is among the positions that may leave.
"""
from __future__ import annotations

import math
from itertools import combinations


def _dot(a, b):
    return sum(float(x) * float(y) for x, y in zip(a, b))


def brute_run(Q, K, V, q_dec, k_dec, v_dec, k_heavy: int, k_recent: int, scale: float,
              policy: str = "accumulated"):
    """Replay prefill plus len(q_dec) decode steps for ONE head.

    Returns a dict with ``colsum`` (prompt column sums), ``kept`` (positions
    alive after prefill), ``outs`` (one output vector per decode step),
    ``evicted`` (evicted position per step, -1 if none), ``alive`` (final set
    of cached positions) and ``acc`` (accumulated score per position).
    """
    n, T = len(Q), len(q_dec)
    k = k_heavy + k_recent
    keys = [list(map(float, r)) for r in K] + [list(map(float, r)) for r in k_dec]
    vals = [list(map(float, r)) for r in V] + [list(map(float, r)) for r in v_dec]
    d = len(keys[0]) if keys else 0
    acc = [0.0] * (n + T)
    seen = [0] * (n + T)  # number of queries that attended to each position

    def worth(j):
        if policy == "accumulated":
            return acc[j]
        if policy == "averaged":
            return acc[j] / seen[j]
        if policy == "position":
            return -float(j)
        raise ValueError(policy)

    # Prefill: every prompt query attends over all prompt keys up to itself.
    for i in range(n):
        w = [math.exp(scale * _dot(Q[i], keys[j])) for j in range(i + 1)]
        z = sum(w)
        for j in range(i + 1):
            acc[j] += w[j] / z
            seen[j] += 1
    colsum = acc[:n]

    if n <= k:
        alive = set(range(n))
    else:
        recent = set(range(n - k_recent, n))
        cand = range(n - k_recent)
        # Largest total value; among equal totals prefer later positions.
        best = max(combinations(cand, k_heavy),
                   key=lambda S: (sum(worth(j) for j in S), sorted(S, reverse=True)))
        alive = set(best) | recent
    kept = set(alive)

    outs, evicted = [], []
    for step in range(T):
        t = n + step
        members = sorted(alive) + [t]
        w = [math.exp(scale * _dot(q_dec[step], keys[j])) for j in members]
        z = sum(w)
        probs = [x / z for x in w]
        outs.append([sum(probs[a] * vals[j][c] for a, j in enumerate(members)) for c in range(d)])
        for a, j in enumerate(members):
            acc[j] += probs[a]
            seen[j] += 1
        if len(alive) < k:
            alive.add(t)
            evicted.append(-1)
            continue
        S = alive | {t}
        leavers = [v for v in S if v <= t - k_recent]

        def total_without(v):
            return sum(worth(u) for u in S if u != v)

        # Largest remaining total; on equal totals the older position leaves.
        out_pos = max(leavers, key=lambda v: (total_without(v), -v))
        alive = S - {out_pos}
        evicted.append(out_pos)

    return dict(colsum=colsum, kept=kept, outs=outs, evicted=evicted, alive=alive, acc=acc)
