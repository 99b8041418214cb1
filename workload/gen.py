"""Seeded synthetic inputs for the H2O fixed-budget KV-cache path.

This module only draws and rounds random numbers. It holds none of the
method's arithmetic (no attention, no scores, no selection), so that both the
fp64 oracle and the GPU path can consume exactly the same inputs.

Structure of the inputs
-----------------------
The H2O page (summary of arXiv 2306.14048v3, section 3.2 "Heavy-Hitters for
Low Miss Rate") reports that accumulated attention follows a power law, with
a few heavy-hitter tokens collecting most of it. Trained weights are not
available here, so a synthetic generator reproduces that structure:

* one fixed unit vector ``u`` per run (a normalised N(0, I_d) draw);
* queries  ``q = N(0, I_d) + 2 u`` (every query leans towards ``u``);
* keys     ``k = N(0, I_d) + s u`` with ``s = min(U**(-1/alpha), 4)``, a
  Pareto type-I draw (x_m = 1) clipped to 4, so a heavy tail of keys aligns
  with ``u`` and keeps attracting attention step after step;
* values   ``v = N(0, I_d)``;
* optionally a sink offset ``+ sink * u`` added to the key at position 0.

Streams
-------
Every flattened head ``g = b * H + h`` owns four independent PCG64 streams
(derived with ``SeedSequence(seed, spawn_key=(kind, g))``): prompt normals,
prompt Pareto uniforms, decode normals, decode Pareto uniforms.  ``u`` comes
from ``spawn_key=(0,)``.  Any subset of heads, and any prefix of decode steps,
can therefore be generated alone and is bit-identical to the same slice of a
full generation.  Arrays are cast once to the K/V dtype (bf16 and fp16 with
round-to-nearest-even) and returned as float32 arrays holding exactly
representable values.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

DTYPES = ("f32", "bf16", "f16")
ELEM_BYTES = {"f32": 4, "bf16": 2, "f16": 2}


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: a single attention layer's decode problem."""

    name: str
    batch: int
    heads: int
    head_dim: int
    dtype: str
    prompt_len: int
    k_heavy: int
    k_recent: int
    steps: int
    alpha: float = 1.5
    sink: float = 0.0
    seed: int = 0

    @property
    def k(self) -> int:
        return self.k_heavy + self.k_recent

    @property
    def n_heads_total(self) -> int:
        return self.batch * self.heads

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    def describe(self) -> str:
        return (f"{self.name}: B={self.batch} H={self.heads} d={self.head_dim} {self.dtype}, "
                f"prompt {self.prompt_len} -> k={self.k} ({self.k_heavy} heavy + {self.k_recent} recent), "
                f"{self.steps} decode steps, pareto alpha={self.alpha}"
                + (f", sink {self.sink}u at position 0" if self.sink else ""))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five synthetic workloads, named by what they are.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 4, 64, "f32", 64, 16, 16, 256, 1.5, 0.0, 1001),
    "opt6.7b_layer": Workload("opt6.7b_layer", 64, 32, 128, "bf16", 1024, 128, 128, 512, 1.5, 0.0, 1002),
    "opt30b_layer": Workload("opt30b_layer", 32, 56, 128, "bf16", 1920, 205, 205, 128, 1.5, 4.0, 1003),
    "long_context": Workload("long_context", 8, 32, 128, "bf16", 16384, 1024, 1024, 256, 1.2, 0.0, 1004),
    "large_batch_f16": Workload("large_batch_f16", 256, 32, 128, "f16", 512, 128, 128, 1024, 1.5, 0.0, 1005),
}


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to ``dtype`` (round-to-nearest-even); return float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        b = x.view(np.uint32)
        lsb = (b >> np.uint32(16)) & np.uint32(1)
        r = (b + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
        return r.view(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def unit_vector(wl: Workload, seed: int | None = None) -> np.ndarray:
    """The run's fixed direction ``u`` (float32, unit norm)."""
    seed = wl.seed if seed is None else seed
    u = _rng(seed, 0).standard_normal(wl.head_dim)
    return (u / np.linalg.norm(u)).astype(np.float32)


def _pareto_clipped(rng: np.random.Generator, count: int, alpha: float) -> np.ndarray:
    uni = 1.0 - rng.random(count)  # in (0, 1]
    return np.minimum(uni ** (-1.0 / alpha), 4.0).astype(np.float32)


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _heads(wl: Workload, heads) -> np.ndarray:
    if heads is None:
        return np.arange(wl.n_heads_total)
    heads = np.asarray(heads, dtype=np.int64).reshape(-1)
    if heads.size and (heads.min() < 0 or heads.max() >= wl.n_heads_total):
        raise ValueError("head index out of range")
    return heads


def make_prompt(wl: Workload, heads=None, seed: int | None = None):
    """Prompt Q, K, V for the given flattened heads: three [G, n, d] float32 arrays."""
    seed = wl.seed if seed is None else seed
    heads = _heads(wl, heads)
    u = unit_vector(wl, seed)
    n, d = wl.prompt_len, wl.head_dim
    Q = np.empty((heads.size, n, d), np.float32)
    K = np.empty_like(Q)
    V = np.empty_like(Q)

    def one(i):
        g = int(heads[i])
        z = _rng(seed, 1, g).standard_normal((n, 3, d), dtype=np.float32)
        s = _pareto_clipped(_rng(seed, 2, g), n, wl.alpha)
        q = z[:, 0] + 2.0 * u
        k = z[:, 1] + s[:, None] * u
        if wl.sink and n > 0:
            k[0] += wl.sink * u
        Q[i] = round_to_dtype(q, wl.dtype)
        K[i] = round_to_dtype(k, wl.dtype)
        V[i] = round_to_dtype(z[:, 2], wl.dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(heads.size)))
    return Q, K, V


def make_decode(wl: Workload, heads=None, steps: int | None = None, seed: int | None = None):
    """Decode-step inputs q, k_new, v_new for the first ``steps`` steps: [G, T, d] float32."""
    seed = wl.seed if seed is None else seed
    heads = _heads(wl, heads)
    steps = wl.steps if steps is None else steps
    if steps < 0 or steps > wl.steps:
        raise ValueError("steps out of range")
    u = unit_vector(wl, seed)
    d = wl.head_dim
    q_out = np.empty((heads.size, steps, d), np.float32)
    k_out = np.empty_like(q_out)
    v_out = np.empty_like(q_out)

    def one(i):
        g = int(heads[i])
        z = _rng(seed, 3, g).standard_normal((steps, 3, d), dtype=np.float32)
        s = _pareto_clipped(_rng(seed, 4, g), steps, wl.alpha)
        q_out[i] = round_to_dtype(z[:, 0] + 2.0 * u, wl.dtype)
        k_out[i] = round_to_dtype(z[:, 1] + s[:, None] * u, wl.dtype)
        v_out[i] = round_to_dtype(z[:, 2], wl.dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(heads.size)))
    return q_out, k_out, v_out


def sample_heads(wl: Workload, count: int, seed: int = 7) -> np.ndarray:
    """A fixed, seeded, sorted subset of flattened head indices (all heads if count >= total)."""
    total = wl.n_heads_total
    if count >= total:
        return np.arange(total)
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(total, size=count, replace=False))
