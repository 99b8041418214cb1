"""Pins of the oracle's quantised cache, 8-, 4- and 2-bit codes (CPU only).

The quantiser is pinned by values worked out by hand (grids with exact
scales, round-half-even ties, clamping, a constant row, packed bytes) and by
its error bound; the quantised H2O oracle is pinned against the plain one, which the
brute-force and closed-form pins already hold: on inputs that lie exactly on
their grids (per channel for keys, per row for values) quantisation is
lossless and the two must agree bit for bit, and a new token attends at full
precision in its own step.
"""
import numpy as np
import pytest

from oracle import H2OOracle
from oracle import quant as qz


def test_codes_on_an_exact_grid():
    scale, mn = qz.row_grid(np.array([0.0, 255.0], np.float32))
    assert scale == 1.0 and mn == 0.0
    x = np.array([0, 1.5, 2.5, 126.5, 127.5, 254.5, 255, -3, 300], np.float32)
    # round half to even; values outside the grid clamp to its ends
    assert qz.quantize(x, scale, mn).tolist() == [0, 2, 2, 126, 128, 254, 255, 0, 255]
    scale, mn = qz.row_grid(np.array([-10.0, 500.0], np.float32))  # 510 / 255 = 2
    assert scale == 2.0 and mn == -10.0
    assert qz.quantize(np.array([-7, -5, 0, 499], np.float32), scale, mn).tolist() == [2, 2, 5, 254]
    assert qz.dequantize(np.array([0, 5, 255], np.uint8), scale, mn).tolist() == [-10.0, 0.0, 500.0]


def test_constant_row_and_channel():
    scale, mn = qz.row_grid(np.full(8, 7.0, np.float32))
    assert scale == 0.0 and mn == 7.0
    codes = qz.quantize(np.full(8, 7.0, np.float32), scale, mn)
    assert codes.tolist() == [0] * 8
    assert np.all(qz.dequantize(codes, scale, mn) == 7.0)
    ks, km = qz.channel_grid(np.array([[1.0, 2.0], [1.0, 6.0]], np.float32))
    assert ks.tolist() == [0.0, np.float32(4.0) / np.float32(255)] and km.tolist() == [1.0, 2.0]


def test_error_bound_and_ends():
    rng = np.random.default_rng(5)
    V = (rng.standard_normal((200, 128)) * rng.uniform(0.1, 10, (200, 1))).astype(np.float32)
    s, m = qz.row_grid(V)
    c = qz.quantize(V, s[:, None], m[:, None])
    err = np.abs(qz.dequantize(c, s[:, None], m[:, None]) - V)
    assert np.all(err <= s[:, None] * (0.5 + 1e-5))
    assert np.all(c[np.arange(200), V.argmin(1)] == 0)
    assert np.all(c[np.arange(200), V.argmax(1)] == 255)
    K = rng.standard_normal((300, 64)).astype(np.float32)
    ks, km = qz.channel_grid(K)
    kc = qz.quantize(K, ks, km)
    assert np.all(np.abs(qz.dequantize(kc, ks, km) - K) <= ks * (0.5 + 1e-5))
    assert np.all(kc.min(0) == 0) and np.all(kc.max(0) == 255)


def test_codes_on_exact_4_and_2_bit_grids():
    scale, mn = qz.grid(0.0, 15.0, 4)
    assert scale == 1.0 and mn == 0.0
    x = np.array([0, 1.5, 2.5, 7.5, 14.5, 15, -3, 30], np.float32)
    assert qz.quantize(x, scale, mn, 4).tolist() == [0, 2, 2, 8, 14, 15, 0, 15]
    scale, mn = qz.grid(-10.0, 20.0, 4)  # 30 / 15 = 2
    assert scale == 2.0
    assert qz.quantize(np.array([-7, -5, 0, 19], np.float32), scale, mn, 4).tolist() == [2, 2, 5, 14]
    scale, mn = qz.grid(0.0, 3.0, 2)
    assert scale == 1.0
    x = np.array([0, 0.5, 1.5, 2.5, 3, 5, -1], np.float32)
    assert qz.quantize(x, scale, mn, 2).tolist() == [0, 0, 2, 2, 3, 3, 0]
    scale, mn = qz.grid(-3.0, 6.0, 2)  # 9 / 3 = 3
    assert scale == 3.0
    assert qz.quantize(np.array([-1.5, 0, 3, 7.5], np.float32), scale, mn, 2).tolist() == [0, 1, 2, 3]
    assert qz.dequantize(np.array([0, 1, 3], np.uint8), scale, mn).tolist() == [-3.0, 0.0, 6.0]
    with pytest.raises(ValueError):
        qz.levels(3)


def test_packed_bytes_by_hand():
    # 4 bits: the lower channel in the low nibble
    assert qz.pack(np.array([[1, 2, 15, 0]], np.uint8), 4).tolist() == [[0x21, 0x0F]]
    # 2 bits: channel c at bit offset 2 * (c % 4)
    assert qz.pack(np.array([1, 2, 3, 0, 0, 0, 0, 3], np.uint8), 2).tolist() == [0x39, 0xC0]
    # 8 bits: one byte per code
    c8 = np.array([7, 200, 0, 255], np.uint8)
    assert qz.pack(c8, 8).tolist() == c8.tolist()
    rng = np.random.default_rng(3)
    for bits in (8, 4, 2):
        c = rng.integers(0, qz.levels(bits) + 1, (5, 3, 64)).astype(np.uint8)
        p = qz.pack(c, bits)
        assert p.shape == (5, 3, 64 * bits // 8)
        assert np.array_equal(qz.unpack(p, bits), c)


@pytest.mark.parametrize("bits", [4, 2])
def test_low_bit_error_bound_and_ends(bits):
    L = qz.levels(bits)
    rng = np.random.default_rng(6 + bits)
    V = (rng.standard_normal((150, 64)) * rng.uniform(0.1, 10, (150, 1))).astype(np.float32)
    s, m = qz.row_grid(V, bits)
    assert np.all(s == (V.max(1) - V.min(1)) / np.float32(L))
    c = qz.quantize(V, s[:, None], m[:, None], bits)
    assert c.max() <= L
    err = np.abs(qz.dequantize(c, s[:, None], m[:, None]) - V)
    assert np.all(err <= s[:, None] * (0.5 + 1e-5))
    assert np.all(c[np.arange(150), V.argmin(1)] == 0)
    assert np.all(c[np.arange(150), V.argmax(1)] == L)
    K = rng.standard_normal((300, 64)).astype(np.float32)
    ks, km = qz.channel_grid(K, bits)
    kc = qz.quantize(K, ks, km, bits)
    assert np.all(np.abs(qz.dequantize(kc, ks, km) - K) <= ks * (0.5 + 1e-5))
    assert np.all(kc.min(0) == 0) and np.all(kc.max(0) == L)


def _grid_inputs(rng, G, n, T, d, bits=8):
    """Keys on per-channel grids with power-of-two steps fixed by the prompt
    (every channel's prompt column holds codes 0 and L); values on per-row
    grids (every row holds codes 0 and L)."""
    L = qz.levels(bits)
    step = 2.0 ** rng.integers(-6, -2, (G, 1, d))
    base = step * rng.integers(-200, -100, (G, 1, d))
    kc = rng.integers(0, L + 1, (G, n + T, d))
    kc[:, 0], kc[:, 1] = 0, L
    K = base + step * kc
    vstep = 2.0 ** rng.integers(-6, -2, (G, n + T, 1))
    vc = rng.integers(0, L + 1, (G, n + T, d))
    vc[..., 0], vc[..., 1] = 0, L
    V = vstep * (vc - rng.integers(100, 200, (G, n + T, 1)))
    Q = rng.standard_normal((G, n + T, d))
    return Q, K, V


@pytest.mark.parametrize("quant", ["u8", "u4", "u2"])
@pytest.mark.parametrize("policy,kh,kr", [("accumulated", 5, 4), ("averaged", 3, 3), ("accumulated", 6, 0)])
def test_quantised_equals_plain_on_grid_inputs(policy, kh, kr, quant):
    rng = np.random.default_rng(11)
    G, n, T, d = 3, 20, 25, 16
    Q, K, V = _grid_inputs(rng, G, n, T, d, qz.BITS[quant])
    scale = 0.3
    plain = H2OOracle(G, d, kh, kr, scale, policy)
    qo = H2OOracle(G, d, kh, kr, scale, policy, quant=quant)
    a, b = plain.prefill(Q[:, :n], K[:, :n], V[:, :n]), qo.prefill(Q[:, :n], K[:, :n], V[:, :n])
    assert np.array_equal(a.colsum, b.colsum)
    assert np.array_equal(plain.K, qo.K) and np.array_equal(plain.V, qo.V)
    for t in range(T):
        i = n + t
        sa = plain.decode_step(Q[:, i], K[:, i], V[:, i])
        sb = qo.decode_step(Q[:, i], K[:, i], V[:, i])
        assert np.array_equal(sa.evicted, sb.evicted)
        assert np.array_equal(sa.out, sb.out)
        assert np.array_equal(plain.score, qo.score) and np.array_equal(plain.pos, qo.pos)
    assert np.array_equal(plain.K, qo.K) and np.array_equal(plain.V, qo.V)
    assert qo.Kq.max() <= qz.levels(qz.BITS[quant]) and qo.Vq.max() <= qz.levels(qz.BITS[quant])


@pytest.mark.parametrize("quant", ["u8", "u4", "u2"])
def test_new_token_attends_at_full_precision_then_is_quantised(quant):
    bits = qz.BITS[quant]
    L = qz.levels(bits)
    rng = np.random.default_rng(12)
    G, n, d = 2, 12, 16
    Q, K, V = _grid_inputs(rng, G, n, 1, d, bits)
    plain = H2OOracle(G, d, 4, 4, 0.25)
    qo = H2OOracle(G, d, 4, 4, 0.25, quant=quant)
    plain.prefill(Q[:, :n], K[:, :n], V[:, :n])
    qo.prefill(Q[:, :n], K[:, :n], V[:, :n])
    # an off-grid new token, its key partly outside the prompt's channel range
    k_new = rng.standard_normal((G, d)) * 3
    k_new[:, 0] = 1e3
    v_new = rng.standard_normal((G, d))
    q = rng.standard_normal((G, d))
    sa, sb = plain.decode_step(q, k_new, v_new), qo.decode_step(q, k_new, v_new)
    assert np.array_equal(sa.out, sb.out) and np.array_equal(sa.evicted, sb.evicted)
    for g in range(G):
        s = sb.slot[g]
        kmax = (qo.k_min[g].astype(np.float64) + L * qo.k_scale[g].astype(np.float64))
        assert qo.Kq[g, s, 0] == L and qo.K[g, s, 0] == kmax[0]  # clamped to the grid's top
        assert np.all(np.abs(qo.K[g, s] - np.clip(k_new[g], qo.k_min[g], kmax))
                      <= qo.k_scale[g] * (0.5 + 1e-5))
        assert np.all(np.abs(qo.V[g, s] - v_new[g]) <= qo.v_scale[g, s] * (0.5 + 1e-5) + 1e-6)


@pytest.mark.parametrize("quant", ["u8", "u4", "u2"])
def test_quantised_cache_needs_a_prompt(quant):
    o = H2OOracle(1, 16, 2, 2, 0.25, quant=quant)
    with pytest.raises(ValueError):
        o.prefill(np.zeros((1, 0, 16)), np.zeros((1, 0, 16)), np.zeros((1, 0, 16)))


def test_unknown_format_rejected():
    with pytest.raises(ValueError):
        H2OOracle(1, 16, 2, 2, 0.25, quant="u3")
