"""Plain float64 CPU oracle of the Heavy-Hitter Oracle (H2O) fixed-budget KV cache.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import or run anything under ``oracle/``. The product path
(the HIP library and its Python binding) never does, and the two share no
code: the only thing both consume is the seeded input generator in
``workload/``, which holds none of the method's arithmetic.

Citations
---------
"H2O §x" means the page "H2O: Heavy-Hitter Oracle for Efficient Generative
Inference of Large Language Models" (the paperlayer.ai source-linked summary
of arXiv 2306.14048v3), section x and the bullet named after it.

What is computed (per (batch, head), independently, all in float64)
------------------------------------------------------------------
Prefill over a prompt of n tokens:
  P[i, j] = softmax over j <= i of scale * <Q_i, K_j>   (H2O §D "Recursive attention")
  c_j     = sum_i P[i, j]                                (accumulated attention, H2O §1, §4.1)
  keep all n tokens when n <= k; otherwise keep the k_recent newest positions
  and the k_heavy candidates in [0, n - k_recent) with the largest (c_j, j)
  (H2O §A "Pseudocode", "System Details").
Decode step at position t:
  attend over the cached tokens plus the new token itself (H2O §D, attention is
  taken over the prefix including row t, before eviction); add each cached
  token's probability to its score (accumulated, not averaged: H2O §B.2
  "Previous Attempts"); when the cache is full, evict the eligible slot with
  the smallest (score, pos), where eligible means pos <= t - k_recent
  (at most one eviction per step, fixed size k: H2O §2 "Problem formulation",
  §D "Cache eviction"); write the new token into the freed slot with score
  p_new.

Readings where the page is silent (the design notes list them all):
  self-attention of the new token is included; accumulation happens before the
  victim is chosen; the recent window is (t - k_recent, t]; the new token's
  initial score is its own probability; ties are broken by the total order
  (score, pos); prefill candidates exclude the recent window; the slot layout is
  heavy positions ascending in slots [0, k_heavy), recent positions ascending in
  [k_heavy, k), and a decode step writes into the victim's slot (or slot n_used
  while the cache is not yet full).

Policies (the variants the page compares H2O with or reports as worse):
  "accumulated" (H2O): a token's value is its accumulated score;
  "averaged": its accumulated score divided by the number of queries that
      have attended to it so far (H2O §B.2 "Previous Attempts" reports this
      variant as worse);
  "position": its value is minus its position, so the earliest tokens stay
      (attention sinks) and the oldest token outside them leaves, which is
      StreamingLLM's sink-plus-window cache (Discoveries (cursor 150),
      StreamingLLM abstract; compared in H2O §C.1 "Long-context generation").
  k_heavy = 0 is the "Local" recent-window baseline and k_recent = 0 the
  heavy-hitter-only ablation (H2O §5 "Ablation and Extended Evaluations");
  with k_recent = 0 the new token itself competes and may be the one evicted.

Quantised cache (quant="u8", "u4" or "u2", oracle/quant.py): cached keys and
values are held as 8-, 4- or 2-bit codes, keys on per-channel grids fixed by
the prompt, values on per-token grids (the KIVI finding in Discoveries (cursor
150); H2O combined with quantisation, H2O §5). Attention reads the dequantised rows; the new
token attends to its own key and value at full precision and is quantised
when it is written into its slot. Scores, selection and eviction are as
above. An empty prompt leaves nothing to calibrate the key grids on, so a
quantised cache needs a prompt of at least one token.

Pins: brute force on tiny inputs, the q = 0 closed form, textbook special
cases (full cache = causal attention, k_heavy = 0 = sliding window, the
position policy = sink-plus-window attention), the budget-3 illustration of
H2O §4.1 and invariants; see tests/test_oracle_pins.py.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import quant as qz


def _over_heads(G: int, workers: int, fn) -> None:
    """Call fn(heads) for contiguous head ranges covering range(G), on up to
    `workers` threads with BLAS single-threaded inside them. Heads are
    independent, so the results are those of one call over all heads."""
    if workers <= 1 or G <= 1:
        fn(slice(0, G))
        return
    from concurrent.futures import ThreadPoolExecutor
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1, user_api="blas")
    except Exception:  # threadpoolctl missing: BLAS keeps its own threads
        limit = None
    try:
        parts = min(workers, G)
        with ThreadPoolExecutor(parts) as ex:
            list(ex.map(lambda i: fn(slice(i * G // parts, (i + 1) * G // parts)), range(parts)))
    finally:
        if limit is not None:
            limit.restore_original_limits()

__all__ = ["causal_attention_probs", "causal_attention_probs_rows", "prefill_column_sums", "prefill_attention", "select_prefill", "retention_value",
           "eligible_slots", "choose_victim", "H2OOracle", "PrefillResult", "StepResult", "POLICIES"]

POLICIES = ("accumulated", "averaged", "position")


def retention_value(score, pos, t, policy: str):
    """How much a cached token is worth keeping at step t (larger = keep).

    accumulated: the accumulated score (H2O §1, §4.1); averaged: that score
    over the number of queries t - pos + 1 that have attended to the token
    (H2O §B.2); position: -pos (earliest tokens are kept, StreamingLLM).
    """
    score = np.asarray(score, np.float64)
    pos = np.asarray(pos)
    if policy == "accumulated":
        return score
    if policy == "averaged":
        return score / (t - pos + 1)
    if policy == "position":
        return -pos.astype(np.float64)
    raise ValueError(f"unknown policy {policy!r}")


def causal_attention_probs(Q: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """Row-softmax attention of every prompt query over the keys up to its own position.

    H2O §D "Recursive attention": query row i attends over the first i key rows
    (its own included) and is normalised by that row's own sum D_i.
    Returns P with P[i, j] = 0 for j > i.
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    n = Q.shape[0]
    S = scale * (Q @ K.T)
    S = np.where(np.tril(np.ones((n, n), dtype=bool)), S, -np.inf)
    E = np.exp(S - S.max(axis=1, keepdims=True))
    return E / E.sum(axis=1, keepdims=True)


def prefill_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """The prompt's own causal attention: output rows O_i = sum_j P[i, j] V_j
    and each row's log normaliser lse_i = log sum_{j <= i} exp(scale <Q_i, K_j>)
    (natural log), H2O §D "Recursive attention" (o_i and D_i)."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    n = Q.shape[0]
    if n == 0:
        return np.zeros((0, V.shape[1])), np.zeros(0)
    S = scale * (Q @ K.T)
    S = np.where(np.tril(np.ones((n, n), dtype=bool)), S, -np.inf)
    mx = S.max(axis=1, keepdims=True)
    E = np.exp(S - mx)
    Z = E.sum(axis=1, keepdims=True)
    return (E / Z) @ V, (mx + np.log(Z))[:, 0]


def prefill_column_sums(Q: np.ndarray, K: np.ndarray, scale: float, block: int = 1024) -> np.ndarray:
    """c_j: total normalised attention that prompt token j receives from all prompt queries.

    This is the accumulated attention statistic of H2O §1 ("Greedy algorithm for
    low-cost policy") and §4.1, taken over the whole prompt (diagonal included).
    The query rows are taken `block` at a time: each row's softmax is complete
    within its block (H2O §D "Recursive attention": row i is normalised by its
    own D_i), so c is the sum of the blocks' column sums and memory stays at
    block x n values whatever the prompt length.
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    n = Q.shape[0]
    c = np.zeros(n, np.float64)
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        c[:r1] += causal_attention_probs_rows(Q[r0:r1], K[:r1], scale, r0).sum(axis=0)
    return c


def causal_attention_probs_rows(Qb: np.ndarray, K: np.ndarray, scale: float, r0: int) -> np.ndarray:
    """Rows r0 .. r0 + len(Qb) - 1 of the causal attention matrix, over keys 0 .. len(K) - 1
    (row i attends over keys j <= i, H2O §D "Recursive attention")."""
    rows = np.arange(r0, r0 + Qb.shape[0])[:, None]
    S = scale * (Qb @ K.T)
    S = np.where(np.arange(K.shape[0])[None, :] <= rows, S, -np.inf)
    E = np.exp(S - S.max(axis=1, keepdims=True))
    return E / E.sum(axis=1, keepdims=True)


def select_prefill(c: np.ndarray, k_heavy: int, k_recent: int, policy: str = "accumulated"):
    """Positions kept after prefill, in slot order, and the selection margin.

    H2O §A "Pseudocode": a prompt long enough is reduced to heavy hitters plus
    recent tokens; §A "System Details": heavy hitters first, recent tokens last.
    Candidates for the heavy part are the positions before the recent window;
    they are ranked by (retention value at the last prompt row, position), so
    on equal values the later position is kept. The margin is the relative
    gap between the smallest kept candidate value and the largest dropped one
    (inf when nothing is dropped or the values cannot tie).
    """
    c = np.asarray(c, np.float64)
    n = c.shape[0]
    k = k_heavy + k_recent
    if n <= k:
        return np.arange(n, dtype=np.int64), np.inf
    recent = np.arange(n - k_recent, n, dtype=np.int64)
    candidates = np.arange(n - k_recent)
    val = retention_value(c[candidates], candidates, n - 1, policy)
    ranked = sorted(range(candidates.size), key=lambda j: (val[j], j), reverse=True)
    heavy = np.array(sorted(ranked[:k_heavy]), dtype=np.int64)
    margin = np.inf
    if 0 < k_heavy < len(ranked) and policy != "position":
        lo_kept, hi_dropped = val[ranked[k_heavy - 1]], val[ranked[k_heavy]]
        margin = (lo_kept - hi_dropped) / lo_kept if lo_kept > 0 else 0.0
    return np.concatenate([heavy, recent]), margin


def eligible_slots(pos: np.ndarray, t: int, k_recent: int) -> np.ndarray:
    """Slots that may be evicted at step t: those outside the recent window (t - k_recent, t].

    H2O §A "System Details" keeps the newest tokens in a recent region; with the
    new token t counted in it, a slot is evictable iff pos <= t - k_recent.
    """
    return (pos >= 0) & (pos <= t - k_recent)


def choose_victim(value: np.ndarray, pos: np.ndarray, eligible: np.ndarray, exact: bool = False):
    """Per head, the eligible candidate with the smallest (value, pos), and the eviction margin.

    H2O §4.1 and §D "Cache eviction": the lowest accumulated score leaves.
    Ties on the value evict the older position. The margin is
    (second smallest - smallest) / second smallest over the eligible values
    (inf when `exact`: the values are distinct integers).
    """
    G = value.shape[0]
    masked = np.where(eligible, value, np.inf)
    smallest = masked.min(axis=1)
    tied = eligible & (value == smallest[:, None])
    victim = np.argmin(np.where(tied, pos, np.iinfo(np.int64).max), axis=1)
    margin = np.full(G, np.inf)
    if not exact and value.shape[1] >= 2:
        e = np.sort(masked, axis=1)  # the eligible values first, ascending
        e0, e1 = e[:, 0], e[:, 1]
        two = eligible.sum(axis=1) >= 2
        gap = np.divide(e1 - e0, e1, out=np.zeros(G), where=two & (e1 > 0))
        margin = np.where(two, gap, np.inf)
    return victim, margin


@dataclass
class PrefillResult:
    colsum: np.ndarray   # [G, n] float64 prompt column sums
    margin: np.ndarray   # [G] selection margin (inf = unique by construction)


@dataclass
class StepResult:
    out: np.ndarray      # [G, d] attention output of the new query
    evicted: np.ndarray  # [G] evicted position, -1 when nothing was evicted
    margin: np.ndarray   # [G] eviction margin (inf when nothing was evicted)
    probs: np.ndarray    # [G, n_used + 1] probabilities over the cached slots then the new token
    slot: np.ndarray     # [G] slot the new token was written into, -1 if it was the one evicted


class H2OOracle:
    """fp64 state of G independent (batch, head) caches with k = k_heavy + k_recent slots.

    State per head: K, V rows per slot, the accumulated score per slot, the
    position each slot holds (-1 = empty), plus the shared counters n_used (the
    number of occupied slots, always min(k, t)) and t (position of the next
    token). Slots [0, n_used) are the occupied ones.
    """

    def __init__(self, n_heads: int, head_dim: int, k_heavy: int, k_recent: int, scale: float,
                 policy: str = "accumulated", quant: str | None = None, workers: int = 1):
        """workers > 1 evaluates independent heads on that many threads (the
        per-head arithmetic, and so every result, is unchanged)."""
        if k_heavy < 0 or k_recent < 0 or k_heavy + k_recent < 1:
            raise ValueError("need k_heavy >= 0, k_recent >= 0 and k >= 1")
        if policy not in POLICIES:
            raise ValueError(f"unknown policy {policy!r}")
        if quant is not None and quant not in qz.BITS:
            raise ValueError(f"unknown quantisation {quant!r}")
        self.policy = policy
        self.quant = quant
        self.workers = max(1, int(workers))
        self.bits = qz.BITS[quant] if quant else None
        self.G, self.d = n_heads, head_dim
        self.k_heavy, self.k_recent = k_heavy, k_recent
        self.k = k_heavy + k_recent
        self.scale = float(scale)
        self.K = np.zeros((self.G, self.k, self.d))
        self.V = np.zeros((self.G, self.k, self.d))
        self.score = np.zeros((self.G, self.k))
        self.pos = np.full((self.G, self.k), -1, dtype=np.int64)
        self.n_used = 0
        self.t = 0
        if quant:
            # codes of the cached rows and their grids (K and V above hold the dequantised rows)
            self.Kq = np.zeros((self.G, self.k, self.d), np.uint8)
            self.Vq = np.zeros((self.G, self.k, self.d), np.uint8)
            self.k_scale = np.zeros((self.G, self.d), np.float32)
            self.k_min = np.zeros((self.G, self.d), np.float32)
            self.v_scale = np.zeros((self.G, self.k), np.float32)
            self.v_min = np.zeros((self.G, self.k), np.float32)

    def _store_rows(self, g, slots, k_rows, v_rows):
        """Write rows into slots of head g (quantised when the cache is)."""
        if not self.quant:
            self.K[g, slots] = k_rows
            self.V[g, slots] = v_rows
            return
        k_rows32 = np.asarray(k_rows, np.float32)  # float32-exact inputs
        v_rows32 = np.asarray(v_rows, np.float32)
        kc = qz.quantize(k_rows32, self.k_scale[g], self.k_min[g], self.bits)
        vs, vm = qz.row_grid(v_rows32, self.bits)
        vc = qz.quantize(v_rows32, vs[..., None], vm[..., None], self.bits)
        self.Kq[g, slots], self.Vq[g, slots] = kc, vc
        self.v_scale[g, slots], self.v_min[g, slots] = vs, vm
        self.K[g, slots] = qz.dequantize(kc, self.k_scale[g], self.k_min[g])
        self.V[g, slots] = qz.dequantize(vc, vs[..., None], vm[..., None])

    def prefill(self, Q: np.ndarray, K: np.ndarray, V: np.ndarray, workers: int | None = None) -> PrefillResult:
        """Score the prompt and seed the cache (H2O §A "Pseudocode"); Q, K, V are [G, n, d].

        workers (default: the oracle's) > 1 computes the heads' column sums on
        that many threads (the heads are independent; each head's arithmetic
        is unchanged)."""
        workers = self.workers if workers is None else workers
        Q = np.asarray(Q, np.float64)
        K = np.asarray(K, np.float64)
        V = np.asarray(V, np.float64)
        n = Q.shape[1]
        if self.quant and n == 0:
            raise ValueError("a quantised cache needs a prompt of at least one token")
        colsum = np.zeros((self.G, n))
        margin = np.full(self.G, np.inf)
        self.score[:] = 0.0
        self.pos[:] = -1
        self.K[:] = 0.0
        self.V[:] = 0.0
        def column_sums(heads):
            for g in range(self.G)[heads]:
                colsum[g] = prefill_column_sums(Q[g], K[g], self.scale)

        _over_heads(self.G, workers if n else 1, column_sums)
        for g in range(self.G):
            keep, margin[g] = select_prefill(colsum[g], self.k_heavy, self.k_recent, self.policy)
            m = keep.size
            self.pos[g, :m] = keep
            self.score[g, :m] = colsum[g][keep]
            if self.quant:
                self.k_scale[g], self.k_min[g] = qz.channel_grid(K[g], self.bits)
            self._store_rows(g, np.arange(m), K[g][keep], V[g][keep])
        self.n_used = min(n, self.k)
        self.t = n
        return PrefillResult(colsum, margin)

    def decode_step(self, q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray) -> StepResult:
        """One decode step for every head; q, k_new, v_new are [G, d].

        Order (H2O §D "Recursive attention" then "Cache eviction"): attend over
        the cache plus the new token, accumulate the probabilities into the
        scores, then evict at most one slot and store the new token.
        """
        q = np.asarray(q, np.float64)
        k_new = np.asarray(k_new, np.float64)
        v_new = np.asarray(v_new, np.float64)
        nu, G = self.n_used, self.G
        Kc, Vc = self.K[:, :nu], self.V[:, :nu]

        qk = np.empty((G, nu))

        def dots(heads):
            qk[heads] = np.matmul(Kc[heads], q[heads, :, None])[:, :, 0]

        _over_heads(G, self.workers, dots)
        logits = np.concatenate([self.scale * qk, self.scale * (k_new * q).sum(axis=1)[:, None]], axis=1)
        e = np.exp(logits - logits.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        pv = np.empty((G, self.d))

        def weighted(heads):
            pv[heads] = np.matmul(p[heads, None, :nu], Vc[heads])[:, 0, :]

        _over_heads(G, self.workers, weighted)
        out = pv + p[:, nu:nu + 1] * v_new

        self.score[:, :nu] += p[:, :nu]

        rows = np.arange(G)
        if nu < self.k:
            slot = np.full(G, nu, dtype=np.int64)
            evicted = np.full(G, -1, dtype=np.int64)
            margin = np.full(G, np.inf)
            self.n_used = nu + 1
        else:
            # Candidates: the cached slots, plus the new token itself (column k)
            # when there is no recent window to protect it.
            cand_pos = np.concatenate([self.pos, np.full((G, 1), self.t)], axis=1)
            cand_score = np.concatenate([self.score, p[:, nu:nu + 1]], axis=1)
            value = retention_value(cand_score, cand_pos, self.t, self.policy)
            elig = eligible_slots(cand_pos, self.t, self.k_recent)
            if self.k_recent > 0:
                elig[:, self.k] = False
            victim, margin = choose_victim(value, cand_pos, elig, exact=self.policy == "position")
            evicted = cand_pos[rows, victim].copy()
            slot = np.where(victim < self.k, victim, -1)

        ins = slot >= 0
        r, sl = rows[ins], slot[ins]
        if self.quant:
            for g, s_ in zip(r, sl):
                self._store_rows(g, np.array([s_]), k_new[g][None], v_new[g][None])
        else:
            self.K[r, sl] = k_new[r]
            self.V[r, sl] = v_new[r]
        self.pos[r, sl] = self.t
        self.score[r, sl] = p[ins, nu]
        self.t += 1
        return StepResult(out, evicted, margin, p, slot)

    def snapshot(self) -> dict:
        """Copy of the full state (used to resync another implementation)."""
        snap = dict(K=self.K.copy(), V=self.V.copy(), score=self.score.copy(),
                    pos=self.pos.copy(), n_used=self.n_used, t=self.t)
        if self.quant:
            snap.update(Kq=self.Kq.copy(), Vq=self.Vq.copy(), k_scale=self.k_scale.copy(),
                        k_min=self.k_min.copy(), v_scale=self.v_scale.copy(), v_min=self.v_min.copy())
        return snap

    def restore(self, snap: dict) -> None:
        """Put back a state taken with snapshot() (arrays are copied in)."""
        for name, value in snap.items():
            if isinstance(value, np.ndarray):
                getattr(self, name)[...] = value
            else:
                setattr(self, name, value)
