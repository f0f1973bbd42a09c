"""Pins of the 2-bit cold-expert format (oracle/quant.quantize_sym2, pack_crumbs,
oracle/layout.to_device2), of MoE layers with 2-bit experts (oracle/ffn.moe_mixed,
moe_w4a16) and of the width rule (oracle/ffn.bits_apex).

Page "大模型之Dense、MoE与量化", APEX section: commonly used experts in 4 bits, rarely
used ones in 2 bits.  The format is the INT4 g128 structure with two bits: scale amax
(rounded up to binary16), codes clamp(rint(w / s), -2, 1), four per byte."""
import math

import numpy as np
import pytest

from oracle import ffn, layout, quant


def _w(n, k, seed, sigma=0.05):
    return np.random.default_rng(seed).normal(0, sigma, (n, k)).astype(np.float32)


def test_codes_are_the_nearest_of_the_four_levels():
    """Brute force: every code is the nearest of the four codes to w / s (the stored
    scale), ties to the even code."""
    w = _w(48, 512, 1)
    w[3, :128] *= 1e-3
    q, s = quant.quantize_sym2(w)
    s32 = np.repeat(s.astype(np.float32), 128, axis=1)
    codes = np.arange(-2, 2, dtype=np.float64)
    r = (w / s32).astype(np.float64)                                  # fp32 division
    dist = np.abs(r[..., None] - codes)
    best = dist.min(axis=-1)
    ok = (np.abs(r - q) == best)
    assert ok.all()
    assert set(np.unique(q)) <= {-1, 0, 1}


def test_scale_is_amax_rounded_up_and_half_step_bound():
    w = _w(64, 384, 2)
    w[0, :128] = 0.0
    w[1, :128] *= 1e-9           # subnormal binary16 scale
    w[2, 128:256] = 3e-8
    q, s = quant.quantize_sym2(w)
    amax = np.abs(w.reshape(64, 3, 128)).max(axis=2)
    s32 = s.astype(np.float32)
    nz = amax > 0
    # smallest binary16 >= amax: s >= amax and the next binary16 below is < amax
    assert np.all(s32[nz] >= amax[nz])
    below = np.nextafter(s[nz], np.float16(-np.inf)).astype(np.float32)
    assert np.all(below < amax[nz])
    assert np.all(s32[~nz] == 0) and np.all(q.reshape(64, 3, 128)[~nz] == 0)
    # half-step bound (the slack covers the fp32 division)
    wh = quant.dequantize(q, s)
    err = np.abs(w.astype(np.float64) - wh).reshape(64, 3, 128)
    assert np.all(err <= s32.astype(np.float64)[:, :, None] / 2 * (1 + 2.0 ** -20))
    # every group with a normal-range scale reaches a +-1 code (s < amax (1 + 2^-10), so
    # its largest |w| has |w / s| > 1/2); a group below the smallest subnormal's half
    # (the 1e-9-scaled one) rounds to zero codes
    qg = np.abs(q.reshape(64, 3, 128)).max(axis=2)
    normal = s32 >= 2.0 ** -14
    assert normal.sum() > 150 and np.all(qg[normal] == 1)
    assert np.all(qg[amax < 2.0 ** -25] == 0)


def test_ties_round_half_to_even():
    s = np.float32(0.5)              # w = 0.25 -> w / s = 0.5 -> 0; w = -0.25 -> -0 -> 0
    row = np.zeros(128, np.float32)
    row[0], row[1], row[2], row[3] = 0.5, 0.25, -0.25, -0.5
    q, sc = quant.quantize_sym2(row[None, :])
    assert sc[0, 0] == np.float16(0.5)
    assert q[0, :4].tolist() == [1, 0, 0, -1]


def test_pack_round_trip_every_byte():
    b = np.arange(256, dtype=np.uint8)[None, :]
    codes = quant.unpack_crumbs(b, 1024)
    assert np.array_equal(quant.pack_crumbs(codes), b)
    # hand-worked byte: codes (1, -1, 0, -2) -> 01 | 11 << 2 | 00 << 4 | 10 << 6
    assert quant.pack_crumbs(np.array([[1, -1, 0, -2]]))[0, 0] == 0b10001101


def test_size_against_fp16():
    n, k = 2048, 7168
    ratio = quant.packed_bytes2(n, k) / (2 * n * k)
    assert ratio == pytest.approx(1 / 8 + 1 / 128)
    # half the code bytes of the 4-bit format, the same scale bytes
    assert quant.packed_bytes(n, k, False) - quant.packed_bytes2(n, k) == n * k // 4


@pytest.mark.parametrize("gate_up", [False, True])
def test_layout_round_trip(gate_up):
    n, k = 64, 512
    q, s = quant.quantize_sym2(_w(n, k, 3))
    dev = layout.to_device2(quant.pack_crumbs(q), s.view(np.uint16), n, k, gate_up)
    assert len(dev) == layout.device_bytes2(n, k)
    q2, s2 = layout.from_device2(dev, n, k, gate_up)
    assert np.array_equal(q2, q) and np.array_equal(s2, s.view(np.uint16))


def test_layout_hand_placement():
    """Column 17, k = 128 + 32 * 3 + 8 * 2 + 5 (group 1, step 3, quarter 2, element 5):
    block 1, lane 2 * 16 + 1 = 33, word 1, byte 1, field 2 * 1 + 1 = 3 -> byte
    512 * (1 * G + 1) + 8 * 33 + 4 + 1, bits 6..7, value q + 2."""
    n, k = 32, 256
    G = k // 128
    q = np.zeros((n, k), np.int64)
    q[17, 128 + 96 + 16 + 5] = 1
    dev = layout.to_device2(quant.pack_crumbs(q), np.zeros((n, G), np.uint16), n, k, False)
    w = dev[: n * k // 4]
    off = 512 * (1 * G + 1) + 8 * 33 + 4 + 1
    assert (w[off] >> 6) & 3 == 3
    others = np.delete(w, off)
    assert np.all(others == 0b10101010)        # every other element holds d = 2 (q = 0)
    assert w[off] & 0x3F == 0b101010


def _experts(E, H, I, bits, seed):
    rng = np.random.default_rng(seed)
    out = []
    for e in range(E):
        mats = []
        for shape in ((I, H), (I, H), (H, I)):
            m = rng.normal(0, 0.05, shape).astype(np.float32)
            q, s = {2: quant.quantize_sym2, 4: quant.quantize_sym, 8: quant.quantize_sym8}[bits[e]](m)
            mats.append((q.astype(np.int64), s, None))
        out.append(tuple(mats))
    return out


def _brute_w4a16(x_row, gate, up, down):
    deq = lambda qm: quant.dequantize(qm[0], qm[1])
    g = deq(gate) @ x_row
    u = deq(up) @ x_row
    return deq(down) @ (g / (1 + np.exp(-g)) * u)


def _brute_int8(x_row, gate, up, down):
    deq = lambda qm: quant.dequantize(qm[0], qm[1])
    qx, sx = ffn.act_quant_int8(x_row[None, :].astype(np.float32))
    xh = qx[0].astype(np.float64) * np.float64(sx[0])
    g, u = deq(gate) @ xh, deq(up) @ xh
    h = g / (1 + np.exp(-g)) * u
    qh, sh = ffn.act_quant_int8(h[None, :].astype(np.float32))
    return deq(down) @ (qh[0].astype(np.float64) * np.float64(sh[0]))


@pytest.mark.parametrize("mode", ["w4a16", "int8"])
def test_moe_with_two_bit_experts_brute_force(mode):
    """A layer of 2-, 4- (and, with INT8 activations, 8-) bit experts plus a shared
    expert, one token and one choice at a time from the dequantised weights."""
    E, H, I, k, t = 6, 256, 128, 2, 5
    bits = [2, 4, 2, 8 if mode == "int8" else 4, 4, 2, 4]
    mats = _experts(E + 1, H, I, bits, 21)
    rng = np.random.default_rng(22)
    x = rng.normal(0, 1, (t, H)).astype(np.float32)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(t)])
    w = rng.dirichlet(np.ones(k), size=t)
    if mode == "w4a16":
        got = ffn.moe_w4a16(x, lambda e: mats[e], ids, w, shared=mats[E])
        brute = _brute_w4a16
    else:
        got = ffn.moe_mixed(x, lambda e: mats[e], bits, ids, w, shared=mats[E], shared_bits=bits[E])
        brute = _brute_int8
    ref = np.zeros((t, H))
    for r in range(t):
        for j in range(k):
            ref[r] += w[r, j] * brute(x[r].astype(np.float64), *mats[ids[r, j]])
        ref[r] += brute(x[r].astype(np.float64), *mats[E])
    assert np.allclose(got, ref, rtol=1e-9, atol=1e-12)


def test_two_bit_experts_lose_more_than_four_bit():
    """2-bit codes cost accuracy against the real weights: the expert's output error is
    well above the 4-bit one's on the same weights (the reason APEX keeps them for
    rarely used experts)."""
    H, I, t = 256, 128, 16
    rng = np.random.default_rng(23)
    g, u, d = rng.normal(0, 0.05, (I, H)), rng.normal(0, 0.05, (I, H)), rng.normal(0, 0.05, (H, I))
    x = rng.normal(0, 1, (t, H))
    hx = g @ x.T
    exact = (d @ (hx / (1 + np.exp(-hx)) * (u @ x.T))).T
    err = {}
    for b, fn in ((2, quant.quantize_sym2), (4, quant.quantize_sym)):
        m = [(lambda qs: (qs[0].astype(np.int64), qs[1], None))(fn(a.astype(np.float32))) for a in (g, u, d)]
        err[b] = ffn.max_rel_l2(ffn.swiglu_w4a16(x, *m), exact)
    assert err[2] > 2 * err[4]


@pytest.mark.parametrize("E,frac8,cold", [(8, 0.0, 0.25), (16, 0.125, 0.5), (256, 0.05, 0.25), (9, 0.0, 0.0),
                                          (10, 1.0, 1.0)])
def test_bits_apex_brute_force(E, frac8, cold):
    rng = np.random.default_rng(E + 3)
    counts = rng.integers(0, 12, E)
    bits = ffn.bits_apex(counts, frac8, cold)
    total = counts.sum()
    n8 = math.ceil(round(frac8 * E, 9))
    assert sum(b == 8 for b in bits) == n8
    for a in range(E):
        if bits[a] == 8:
            for c in range(E):
                if bits[c] != 8:
                    assert counts[a] > counts[c] or (counts[a] == counts[c] and a < c)
        else:
            assert bits[a] == (2 if counts[a] * E < cold * total else 4)
    assert ffn.bits_apex(counts, frac8, cold, shared=True)[-1] == (8 if frac8 > 0 else 4)


def test_bits_apex_hand_case():
    # total 40 over 4 experts: even share 10; cold below 2.5 hits
    assert ffn.bits_apex([2, 20, 15, 3], 0.0, 0.25) == [2, 4, 4, 4]
    assert ffn.bits_apex([2, 20, 15, 3], 0.25, 0.25, shared=True) == [2, 8, 4, 4, 8]
    assert ffn.bits_apex([0, 0, 0, 0], 0.0, 0.25) == [4, 4, 4, 4]
