"""Pins of the oracle at group sizes other than 128 (32, 64, 256: per-expert group size
by hotness): quantisation by brute force, the half-step bound, a constructed case where
finer groups change nothing, the device layout's scale table (round trip and hand
placement), INT8 group sums and the W4A8 linear against element-by-element evaluation,
the error ordering the finer groups exist for, and the hit-count rule."""
import math

import numpy as np
import pytest

from oracle import ffn, layout, quant


def _w(n, k, seed, sigma=0.05):
    rng = np.random.default_rng(seed)
    w = rng.normal(0.0, sigma, (n, k)).astype(np.float32)
    w[0, :32] *= 1e-3          # a quiet first sub-group
    w[1, 40:50] *= 30.0        # an outlier inside one sub-group
    return w


@pytest.mark.parametrize("group", [32, 64, 256])
def test_sym_codes_and_scales_by_brute_force(group):
    n, k = 8, 512
    w = _w(n, k, group)
    q, s = quant.quantize_sym(w, group)
    assert s.shape == (n, k // group)
    for r in range(n):
        for gi in range(k // group):
            seg = w[r, gi * group:(gi + 1) * group]
            amax = max(abs(float(v)) for v in seg)
            assert s[r, gi] == np.float16(np.float32(amax) / np.float32(7.0))
            sc = float(np.float32(s[r, gi]))
            for j, v in enumerate(seg):
                code = int(q[r, gi * group + j])
                # nearest code in [-8, 7] to v / s (fp32 quotient), ties to even
                t = float(np.float32(v) / np.float32(sc))
                best = min(range(-8, 8), key=lambda c: (abs(t - c), c % 2))
                assert code == best


@pytest.mark.parametrize("group", [32, 64, 128, 256])
def test_half_step_bound_and_dequantize_infers_the_group(group):
    w = _w(16, 1024, 7 + group)
    q, s = quant.quantize_sym(w, group)
    what = quant.dequantize(q, s)
    bound = np.repeat(s.astype(np.float64), group, axis=1) / 2
    assert np.all(np.abs(w.astype(np.float64) - what) <= bound * (1 + 2.0 ** -20))
    qa, sa, za = quant.quantize_asym(w, group)
    whata = quant.dequantize(qa, sa, za)
    bounda = np.repeat(sa.astype(np.float64), group, axis=1) / 2
    assert np.all(np.abs(w.astype(np.float64) - whata) <= bounda * (1 + 2.0 ** -19))


def test_finer_groups_change_nothing_when_every_subgroup_has_the_group_amax():
    rng = np.random.default_rng(3)
    w = rng.uniform(-0.9, 0.9, (4, 256)).astype(np.float32)
    w[:, ::32] = 1.0            # every 32-element sub-group reaches the same amax
    q128, s128 = quant.quantize_sym(w, 128)
    q32, s32 = quant.quantize_sym(w, 32)
    q256, s256 = quant.quantize_sym(w, 256)
    assert np.array_equal(q128, q32) and np.array_equal(q128, q256)
    assert np.array_equal(np.repeat(s128, 4, axis=1), s32)
    assert np.array_equal(s256, s128[:, ::2])


def test_finer_groups_are_closer_to_the_weights():
    w = np.random.default_rng(4).normal(0, 0.02, (64, 2048)).astype(np.float32)
    err = []
    for g in (32, 64, 128, 256):
        q, s = quant.quantize_sym(w, g)
        err.append(float(np.sqrt(np.mean((quant.dequantize(q, s) - w) ** 2))))
    assert err[0] < err[1] < err[2] < err[3]


@pytest.mark.parametrize("group,asym", [(32, False), (64, False), (256, False), (256, True), (128, True)])
@pytest.mark.parametrize("gate_up", [False, True])
def test_layout_round_trip(group, asym, gate_up):
    n, k = 64, 512
    packed, sbits, zp = quant.quantize_pack(_w(n, k, 11), asym, group)
    dev = layout.to_device(packed, sbits, zp, n, k, asym, gate_up, group)
    assert dev.shape[0] == layout.device_bytes(n, k, asym, group)
    q, s, z = layout.from_device(dev, n, k, asym, gate_up, group)
    q0, s0, z0 = quant.unpack_canonical(packed, sbits, zp, k, asym, group)
    assert np.array_equal(q, q0) and np.array_equal(s, s0.view(np.uint16))
    if asym:
        assert np.array_equal(z, z0)


def test_layout_scale_entries_by_hand():
    n, k = 32, 512                       # G = 4 tiles of 128
    w = _w(n, k, 12)
    so = layout._a256(n * k // 2)
    # groups of 32: entry (column block 1, tile 2, j = 3) of column 16 + 5 is at
    # ((1 * 4 + 2) * 16 + 5) * 4 + 3 and holds the scale of k in [2*128 + 96, 2*128 + 128)
    packed, sbits, _ = quant.quantize_pack(w, False, 32)
    dev = layout.to_device(packed, sbits, None, n, k, False, False, 32)
    at = so + 2 * (((1 * 4 + 2) * 16 + 5) * 4 + 3)
    assert int(dev[at]) | (int(dev[at + 1]) << 8) == int(sbits[21, (256 + 96) // 32])
    # groups of 256: tiles 2 and 3 of column 7 both hold the scale of group 1
    packed, sbits, _ = quant.quantize_pack(w, False, 256)
    dev = layout.to_device(packed, sbits, None, n, k, False, False, 256)
    for tile in (2, 3):
        at = so + 2 * ((0 * 4 + tile) * 16 + 7)
        assert int(dev[at]) | (int(dev[at + 1]) << 8) == int(sbits[7, 1])
    # the weight bytes do not depend on the group
    p128, s128, _ = quant.quantize_pack(w, False, 128)
    d128 = layout.to_device(packed, s128, None, n, k, False, False, 128)
    assert np.array_equal(d128[: n * k // 2], dev[: n * k // 2])


@pytest.mark.parametrize("group", [32, 64])
def test_group_acc_and_w4a8_linear_against_elementwise_sums(group):
    rng = np.random.default_rng(group)
    n, k, t = 6, 256, 3
    qm = tuple(v for v in quant.quantize_sym(_w(n, k, 13), group)) + (None,)
    qx = rng.integers(-128, 128, (t, k))
    acc = ffn.group_acc(qx, ffn.widen_int8(qm), group)
    assert acc.shape == (t, n, k // group)
    for a in range(t):
        for c in range(n):
            for gi in range(k // group):
                ref = sum(int(qx[a, kk]) * int(qm[0][c, kk]) for kk in range(gi * group, (gi + 1) * group))
                assert acc[a, c, gi] == ref
    sx = rng.uniform(0.01, 0.1, t).astype(np.float32)
    y = ffn.linear_w4a8(qx, sx, qm)
    wd = quant.dequantize(qm[0], qm[1])
    ref = (qx.astype(np.float64) * sx.astype(np.float64)[:, None]) @ wd.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("E,seed", [(8, 0), (20, 1), (256, 2), (7, 3)])
def test_groups_by_hotness_brute_force(E, seed):
    rng = np.random.default_rng(seed)
    counts = rng.integers(0, 40, E)
    counts[rng.integers(0, E)] = 0
    g = ffn.groups_by_hotness(counts, 0.05, 0.1)
    n_hot = math.ceil(round(0.05 * E, 9))
    assert sum(v == 32 for v in g) == n_hot
    total = int(counts.sum())
    for e in range(E):
        hotter = sum(1 for o in range(E) if counts[o] > counts[e] or (counts[o] == counts[e] and o < e))
        if hotter < n_hot:
            assert g[e] == 32
        elif counts[e] * E < 0.1 * total:
            assert g[e] == 256
        else:
            assert g[e] == 64
    assert ffn.groups_by_hotness(counts, 0.05, 0.1, shared=True) == g + [32]


def test_groups_by_hotness_hand_case():
    # total 100 over 5 experts: even share 20, cold below 2
    assert ffn.groups_by_hotness([50, 1, 30, 19, 0], 0.2, 0.1) == [32, 256, 64, 64, 256]


@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
def test_moe_with_per_expert_groups_against_token_by_token_evaluation(mode):
    """Experts quantised at different group sizes go through the same MoE functions;
    each token is evaluated alone from the dequantised weights."""
    E, H, I, k, t = 4, 256, 256, 2, 5
    groups = [32, 64, 128, 256]
    rng = np.random.default_rng(21)
    mats = []
    for e in range(E):
        m = []
        for shape in ((I, H), (I, H), (H, I)):
            q, s = quant.quantize_sym(rng.normal(0, 0.05, shape).astype(np.float32), groups[e])
            m.append((q.astype(np.int64), s, None))
        mats.append(tuple(m))
    x = rng.normal(0, 1, (t, H)).astype(np.float32)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(t)])
    w = rng.dirichlet(np.ones(k), size=t)
    fn = ffn.moe_w4a16 if mode == "w4a16" else ffn.moe_w4a8
    got = fn(x, lambda e: mats[e], ids, w)
    ref = np.zeros((t, H))
    for r in range(t):
        for j in range(k):
            g, u, d = (quant.dequantize(q, s) for q, s, _ in mats[ids[r, j]])
            if mode == "w4a16":
                xv = x[r].astype(np.float64)
                a, b = g @ xv, u @ xv
                ref[r] += w[r, j] * (d @ (a / (1 + np.exp(-a)) * b))
            else:
                qx, sx = ffn.act_quant_int8(x[r:r + 1])
                xv = qx[0].astype(np.float64) * np.float64(sx[0])
                a, b = g @ xv, u @ xv
                h = a / (1 + np.exp(-a)) * b
                qh, sh = ffn.act_quant_int8(h[None, :].astype(np.float32))
                ref[r] += w[r, j] * (d @ (qh[0].astype(np.float64) * np.float64(sh[0])))
    assert np.allclose(got, ref, rtol=1e-9, atol=1e-12)
