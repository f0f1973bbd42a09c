"""Pins of the W8A8 oracle pieces: INT8 g128 quantisation (oracle/quant.quantize_sym8),
its device layout (oracle/layout.to_device8) and the W8A8 linear (oracle/ffn.linear_w8a8)."""
import numpy as np
import pytest

from oracle import ffn, layout, quant


def _weights(n, k, seed):
    rng = np.random.default_rng(seed)
    w = rng.normal(0.0, 0.02, size=(n, k)).astype(np.float32)
    w[0, :128] *= 1e-3
    w[1, 128:256] *= 1e3
    w[2, :128] = 0.0
    return w


@pytest.mark.parametrize("seed", [0, 1])
def test_codes_are_nearest_by_brute_force(seed):
    w = _weights(32, 512, seed)
    q, s = quant.quantize_sym8(w)
    s64 = np.repeat(s.astype(np.float64), 128, axis=1)
    nz = s64 > 0
    r = w.astype(np.float64)[nz] / s64[nz]
    codes = np.arange(-127, 128, dtype=np.float64)
    best = np.min(np.abs(r[:, None] - codes[None, :]), axis=1)
    assert np.all(np.abs(r - q[nz]) <= best + 1e-5)
    assert np.all(q[~nz] == 0)


def test_half_step_bound_scale_and_extreme_codes():
    w = _weights(64, 1024, 2)
    q, s = quant.quantize_sym8(w)
    what = quant.dequantize(q, s)
    s64 = np.repeat(s.astype(np.float64), 128, axis=1)
    assert np.all(np.abs(w.astype(np.float64) - what) <= s64 / 2 * (1 + 2.0 ** -20))
    amax = np.abs(w.reshape(64, 8, 128)).max(axis=2)
    t = amax / np.float32(127)
    # the stored scale is the smallest binary16 >= amax / 127
    assert np.all(s.astype(np.float32) >= t)
    below = np.nextafter(s, np.float16(0)).astype(np.float32)
    assert np.all((below < t) | (s == 0))
    qa = np.abs(q.reshape(64, 8, 128).astype(np.int64)).max(axis=2)
    normal = s.astype(np.float32) >= 2.0 ** -14
    assert np.all(qa[normal] == 127)                       # normal-range scales reach +-127
    assert q.min() >= -127


def test_exact_ties_round_half_to_even():
    s = np.float16(0.5)
    w = np.zeros((1, 128), dtype=np.float32)
    w[0, 0] = 127 * 0.5                          # amax 63.5 -> s = 0.5 exactly
    w[0, 1] = 2.5 * 0.5                          # 2.5 -> 2
    w[0, 2] = 3.5 * 0.5                          # 3.5 -> 4
    w[0, 3] = -2.5 * 0.5                         # -2.5 -> -2
    q, sc = quant.quantize_sym8(w)
    assert sc[0, 0] == s
    assert q[0, :4].tolist() == [127, 2, 4, -2]


@pytest.mark.parametrize("gate_up", [False, True])
def test_layout8_roundtrip(gate_up):
    w = _weights(64, 384, 3)
    q, s = quant.quantize_sym8(w)
    dev = layout.to_device8(q, s.view(np.uint16), 64, 384, gate_up)
    assert dev.size == layout.device_bytes8(64, 384)
    q2, s2 = layout.from_device8(dev, 64, 384, gate_up)
    assert np.array_equal(q2, q.astype(np.int64)) and np.array_equal(s2, s.view(np.uint16))


def test_layout8_single_element_by_hand():
    # row 17 (block 1, column 1), k = 128 + 64 + 32 + 8 * 2 + 5: tile (1, 1) of a
    # 2-group matrix = tile 3, half 1, upper 8 bytes, lane 2 * 16 + 1 = 33, byte 5
    n, k = 32, 256
    q = np.zeros((n, k), dtype=np.int64)
    q[17, 128 + 64 + 32 + 16 + 5] = -3
    dev = layout.to_device8(q, np.zeros((n, 2), np.uint16), n, k, False)
    off = 3 * 2048 + 1 * 1024 + 33 * 16 + 8 + 5
    assert dev[off] == 0xFD
    assert np.count_nonzero(dev[: n * k]) == 1


def test_w8a8_linear_brute_force():
    rng = np.random.default_rng(5)
    t, n, k = 3, 4, 256
    w = rng.normal(0, 0.05, (n, k)).astype(np.float32)
    q, s = quant.quantize_sym8(w)
    x = rng.normal(size=(t, k)).astype(np.float32)
    qx, sx = ffn.act_quant_int8(x)
    y = ffn.linear_w8a8(qx, sx, (q, s, None))
    for a in range(t):
        for b in range(n):
            ref = 0.0
            for g in range(2):
                acc = 0
                for c in range(128 * g, 128 * g + 128):
                    acc += int(qx[a, c]) * int(q[b, c])
                ref += float(s[b, g]) * acc
            assert y[a, b] == pytest.approx(float(sx[a]) * ref, rel=1e-12, abs=1e-12)


def test_w8a8_closer_to_fp_than_w4a8():
    """8-bit weights: the W8A8 FFN is much closer to the unquantised-weight product than W4A8."""
    rng = np.random.default_rng(6)
    x = rng.normal(size=(8, 256)).astype(np.float32)
    w = rng.normal(0, 0.05, (64, 256)).astype(np.float32)
    qx, sx = ffn.act_quant_int8(x)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    q8, s8 = quant.quantize_sym8(w)
    q4, s4 = quant.quantize_sym(w)
    e8 = ffn.max_rel_l2(ffn.linear_w8a8(qx, sx, (q8, s8, None)), exact)
    e4 = ffn.max_rel_l2(ffn.linear_w4a8(qx, sx, (q4.astype(np.int64), s4, None)), exact)
    assert e8 < 0.02 and e8 < e4 / 3
