"""Plain affine quantisation of the H2O cache's keys and values (oracle side).

TEST INFRASTRUCTURE, like the rest of ``oracle/``: only the tests, the smoke
check and the benchmark's CPU baseline leg use it.

Citations: "Discoveries (cursor 150)" is the attentionhub.org listing page whose
KIVI abstract reports that the key cache should be quantised per channel
(elements of one channel grouped together) and the value cache per token, at
as little as 2 bits; "H2O §5" is the H2O page's "Ablation and Extended
Evaluations" bullet, which reports that H2O combined with quantisation beats
either alone.

Format (one (batch, head) pair), for b = 8, 4 or 2 bits and L = 2^b - 1:
  keys   - per channel c, an affine grid fixed by the prompt: mn_c and
           mx_c are the smallest and largest prompt key values in channel c,
           scale_c = (mx_c - mn_c) / L; every cached key (prompt rows and
           later decode tokens) is stored as codes in channel c's grid, later
           keys clamped to it.
  values - per token, an affine grid over the row's own d values.
  code   = rint((x - mn) / scale) clamped to [0, L], 0 when scale == 0;
  value  = code * scale + mn.
  bytes  - a row of d codes takes d * b / 8 bytes; channel c sits in byte
           c * b // 8 at bit offset b * (c mod (8 / b)), so the low bits of a
           byte hold the lower channel.
All of a code's arithmetic is float32 with IEEE rounding (subtraction, a
correctly rounded division, round-half-even), so another implementation that
does the same float32 operations reaches the same integer codes. The
dequantised values are formed in float64 here.
"""
from __future__ import annotations

import numpy as np

BITS = {"u8": 8, "u4": 4, "u2": 2}  # the storage formats by name


def levels(bits: int) -> int:
    """Largest code of a b-bit grid."""
    if bits not in (8, 4, 2):
        raise ValueError(f"unsupported code width {bits}")
    return (1 << bits) - 1


def grid(lo, hi, bits: int = 8):
    """(scale, mn) of the b-bit grid spanning [lo, hi], in float32."""
    lo = np.asarray(lo, np.float32)
    hi = np.asarray(hi, np.float32)
    return (hi - lo) / np.float32(levels(bits)), lo


def channel_grid(K: np.ndarray, bits: int = 8):
    """Per-channel key grid of one head's prompt keys K [n, d] (n >= 1)."""
    K = np.asarray(K, np.float32)
    return grid(K.min(axis=0), K.max(axis=0), bits)


def row_grid(V: np.ndarray, bits: int = 8):
    """Per-token value grids of rows V [..., d]: one (scale, mn) per row."""
    V = np.asarray(V, np.float32)
    return grid(V.min(axis=-1), V.max(axis=-1), bits)


def quantize(x: np.ndarray, scale: np.ndarray, mn: np.ndarray, bits: int = 8) -> np.ndarray:
    """Codes (one uint8 per element) of x on the grid (scale, mn), float32 arithmetic."""
    x = np.asarray(x, np.float32)
    scale = np.asarray(scale, np.float32)
    mn = np.asarray(mn, np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint((x - mn) / scale)
    q = np.where(scale > 0, q, np.float32(0))
    return np.clip(q, 0, levels(bits)).astype(np.uint8)


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """Bytes of code rows [..., d] in the storage layout: [..., d * bits // 8] uint8."""
    codes = np.asarray(codes, np.uint8)
    per = 8 // bits
    d = codes.shape[-1]
    if d % per:
        raise ValueError("row length must fill whole bytes")
    grouped = codes.reshape(*codes.shape[:-1], d // per, per).astype(np.uint32)
    out = np.zeros(grouped.shape[:-1], np.uint32)
    for i in range(per):
        out |= grouped[..., i] << (bits * i)
    return out.astype(np.uint8)


def unpack(data: np.ndarray, bits: int) -> np.ndarray:
    """Codes [..., d] of packed rows [..., d * bits // 8] (the inverse of pack)."""
    data = np.asarray(data, np.uint8).astype(np.uint32)
    per = 8 // bits
    mask = (1 << bits) - 1
    parts = [(data >> (bits * i)) & mask for i in range(per)]
    return np.stack(parts, axis=-1).reshape(*data.shape[:-1], data.shape[-1] * per).astype(np.uint8)


def dequantize(codes: np.ndarray, scale: np.ndarray, mn: np.ndarray) -> np.ndarray:
    """float64 values code * scale + mn."""
    return np.asarray(codes, np.float64) * np.asarray(scale, np.float64) + np.asarray(mn, np.float64)
