"""Pins of the mixed-width MoE oracle (oracle/ffn.moe_mixed: each expert's weights in
4-bit or 8-bit g128 codes, INT8 activations everywhere) and of the hotness rule that
assigns the widths (oracle/ffn.bits_by_hotness).

The brute-force pin evaluates one token and one choice at a time from the dequantised
weights (codes times scales) and the dequantised activation codes, as plain matrix
products in float64: the grouped INT32 sums of the oracle are an exact regrouping of
that sum, so the two agree to rounding."""
import math

import numpy as np
import pytest

from oracle import ffn, quant


def _qmat(w, bits):
    if bits == 8:
        q, s = quant.quantize_sym8(w)
    else:
        q, s = quant.quantize_sym(w)
    return q.astype(np.int64), s, None


def _experts(E, H, I, bits, seed):
    rng = np.random.default_rng(seed)
    mats = []
    for e in range(E):
        g = rng.normal(0, 0.05, (I, H)).astype(np.float32)
        u = rng.normal(0, 0.05, (I, H)).astype(np.float32)
        d = rng.normal(0, 0.05, (H, I)).astype(np.float32)
        mats.append(tuple(_qmat(m, bits[e]) for m in (g, u, d)))
    return mats


def _dense(qm):
    q, s, _ = qm
    return quant.dequantize(q, s)


def _brute_token(x_row, gate, up, down):
    """One token through one expert from dequantised weights and activations."""
    qx, sx = ffn.act_quant_int8(x_row[None, :].astype(np.float32))
    xh = qx.astype(np.float64) * np.float64(sx[0])
    g = _dense(gate) @ xh[0]
    u = _dense(up) @ xh[0]
    h = g / (1.0 + np.exp(-g)) * u
    qh, sh = ffn.act_quant_int8(h[None, :].astype(np.float32))
    hh = qh.astype(np.float64)[0] * np.float64(sh[0])
    return _dense(down) @ hh


@pytest.mark.parametrize("shared", [False, True])
def test_mixed_moe_against_token_by_token_brute_force(shared):
    E, H, I, k, t = 5, 256, 128, 2, 6
    bits = [8, 4, 4, 8, 4] + ([8] if shared else [])
    mats = _experts(E + int(shared), H, I, bits, 11)
    rng = np.random.default_rng(12)
    x = rng.normal(0, 1, (t, H)).astype(np.float32)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(t)])
    w = rng.dirichlet(np.ones(k), size=t)
    got = ffn.moe_mixed(x, lambda e: mats[e], bits, ids, w, shared=mats[E] if shared else None, shared_bits=8)
    ref = np.zeros((t, H))
    for r in range(t):
        for j in range(k):
            ref[r] += w[r, j] * _brute_token(x[r], *mats[ids[r, j]])
        if shared:
            ref[r] += _brute_token(x[r], *mats[E])
    assert np.allclose(got, ref, rtol=1e-9, atol=1e-12)


def test_uniform_widths_reduce_to_the_uniform_routes():
    E, H, I, k, t = 4, 128, 256, 2, 5
    rng = np.random.default_rng(13)
    x = rng.normal(0, 1, (t, H)).astype(np.float32)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(t)])
    w = rng.dirichlet(np.ones(k), size=t)
    for b, uniform in ((4, ffn.moe_w4a8), (8, ffn.moe_w8a8)):
        mats = _experts(E, H, I, [b] * E, 14)
        got = ffn.moe_mixed(x, lambda e: mats[e], [b] * E, ids, w)
        assert np.array_equal(got, uniform(x, lambda e: mats[e], ids, w))


def test_eight_bit_experts_are_closer_to_the_real_weights():
    """The point of the wider codes: the 8-bit expert's output error against the
    unquantised expert is far below the 4-bit one's on the same weights."""
    H, I, t = 256, 128, 16
    rng = np.random.default_rng(15)
    g, u = rng.normal(0, 0.05, (I, H)), rng.normal(0, 0.05, (I, H))
    d = rng.normal(0, 0.05, (H, I))
    x = rng.normal(0, 1, (t, H)).astype(np.float32)
    hx = (g @ x.T.astype(np.float64))
    exact = (d @ (hx / (1 + np.exp(-hx)) * (u @ x.T.astype(np.float64)))).T
    err = {}
    for b in (4, 8):
        m = [_qmat(a.astype(np.float32), b) for a in (g, u, d)]
        err[b] = ffn.max_rel_l2(ffn.swiglu_int8_acts(x, *m, b), exact)
    assert err[8] < err[4] / 4


@pytest.mark.parametrize("E,frac", [(8, 0.25), (16, 0.05), (256, 0.05), (7, 0.0), (7, 1.0), (10, 0.3)])
def test_bits_by_hotness_brute_force(E, frac):
    rng = np.random.default_rng(E)
    counts = rng.integers(0, 4, E)           # many ties
    bits = ffn.bits_by_hotness(counts, frac)
    n8 = math.ceil(round(frac * E, 9))
    assert sum(b == 8 for b in bits) == n8 and all(b in (4, 8) for b in bits)
    # every 8-bit expert is hit at least as often as every 4-bit one, ties by lower index
    for a in range(E):
        for c in range(E):
            if bits[a] == 8 and bits[c] == 4:
                assert counts[a] > counts[c] or (counts[a] == counts[c] and a < c)
    assert ffn.bits_by_hotness(counts, frac, shared=True) == bits + [8]


def test_bits_by_hotness_hand_case():
    assert ffn.bits_by_hotness([5, 9, 9, 1], 0.5) == [4, 8, 8, 4]
    assert ffn.bits_by_hotness([5, 9, 9, 1], 0.25) == [4, 8, 4, 4]
    assert ffn.bits_by_hotness([0] * 20, 0.05) == [8] + [4] * 19
