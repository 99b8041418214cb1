"""Plain 8-bit quantisation of the H2O cache's keys and values (oracle side).

TEST INFRASTRUCTURE, like the rest of ``oracle/``: only the tests, the smoke
check and the benchmark's CPU baseline leg use it.

Citations: "Discoveries (cursor 150)" is the attentionhub.org listing page whose
KIVI abstract reports that the key cache should be quantised per channel
(elements of one channel grouped together) and the value cache per token;
"H2O §5" is the H2O page's "Ablation and Extended Evaluations" bullet, which
reports that H2O combined with quantisation beats either alone.

Format (one (batch, head) pair):
  keys   - per channel c, an affine grid fixed by the prompt: mn_c and
           mx_c are the smallest and largest prompt key values in channel c,
           scale_c = (mx_c - mn_c) / 255; every cached key (prompt rows and
           later decode tokens) is stored as codes in channel c's grid, later
           keys clamped to it.
  values - per token, an affine grid over the row's own d values.
  code   = rint((x - mn) / scale) clamped to [0, 255], 0 when scale == 0;
  value  = code * scale + mn.
All of a code's arithmetic is float32 with IEEE rounding (subtraction, a
correctly rounded division, round-half-even), so another implementation that
does the same float32 operations reaches the same integer codes. The
dequantised values are formed in float64 here.
"""
from __future__ import annotations

import numpy as np

LEVELS = 255  # codes 0..255


def grid(lo, hi):
    """(scale, mn) of the 8-bit grid spanning [lo, hi], in float32."""
    lo = np.asarray(lo, np.float32)
    hi = np.asarray(hi, np.float32)
    return (hi - lo) / np.float32(LEVELS), lo


def channel_grid(K: np.ndarray):
    """Per-channel key grid of one head's prompt keys K [n, d] (n >= 1)."""
    K = np.asarray(K, np.float32)
    return grid(K.min(axis=0), K.max(axis=0))


def row_grid(V: np.ndarray):
    """Per-token value grids of rows V [..., d]: one (scale, mn) per row."""
    V = np.asarray(V, np.float32)
    return grid(V.min(axis=-1), V.max(axis=-1))


def quantize(x: np.ndarray, scale: np.ndarray, mn: np.ndarray) -> np.ndarray:
    """uint8 codes of x on the grid (scale, mn), float32 arithmetic (broadcasting)."""
    x = np.asarray(x, np.float32)
    scale = np.asarray(scale, np.float32)
    mn = np.asarray(mn, np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint((x - mn) / scale)
    q = np.where(scale > 0, q, np.float32(0))
    return np.clip(q, 0, LEVELS).astype(np.uint8)


def dequantize(codes: np.ndarray, scale: np.ndarray, mn: np.ndarray) -> np.ndarray:
    """float64 values code * scale + mn."""
    return np.asarray(codes, np.float64) * np.asarray(scale, np.float64) + np.asarray(mn, np.float64)
