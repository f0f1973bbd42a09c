"""Pins of the oracle's FFN / MoE forward in W4A16 and W4A8 (CPU only)."""
import math

import numpy as np
import pytest

from oracle import ffn, quant, router


def _rand_w(rng, n, k, sigma=0.05):
    return rng.normal(0, sigma, size=(n, k)).astype(np.float32)


def _qmat(w, asym):
    if asym:
        q, s, z = quant.quantize_asym(w)
        return (q.astype(np.int64), s, z.astype(np.int64))
    q, s = quant.quantize_sym(w)
    return (q.astype(np.int64), s, None)


def _bf16_values(rng, t, h, scale=1.0):
    # bf16-representable values: round float32 to 8 significant bits, half-even
    x = (rng.normal(0, scale, size=(t, h))).astype(np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32)


def _brute_dequant(packed, scale_bits, zeros_packed, n, k, asym):
    """Element-by-element decode of the canonical bytes (independent of quant.dequantize)."""
    out = [[0.0] * k for _ in range(n)]
    for r in range(n):
        for c in range(k):
            byte = int(packed[r, c // 2])
            nib = (byte >> (4 * (c % 2))) & 0xF
            g = c // 128
            s = float(np.uint16(scale_bits[r, g]).view(np.float16))
            if asym:
                zb = int(zeros_packed[r, g // 2])
                z = (zb >> (4 * (g % 2))) & 0xF
                out[r][c] = (nib - z) * s
            else:
                code = nib - 16 if nib >= 8 else nib
                out[r][c] = code * s
    return out


def _brute_ffn(x_row, G, U, D):
    h = []
    for i in range(len(G)):
        g = sum(a * b for a, b in zip(x_row, G[i]))
        u = sum(a * b for a, b in zip(x_row, U[i]))
        h.append(g / (1.0 + math.exp(-g)) * u)
    return [sum(a * b for a, b in zip(h, D[r])) for r in range(len(D))]


@pytest.mark.parametrize("asym,e,k", [(False, 8, 2), (True, 4, 4)])
def test_moe_w4a16_equals_bruteforce_of_every_expert(asym, e, k):
    rng = np.random.default_rng(10 + e)
    t, h, i = 5, 128, 128
    raw = [(_rand_w(rng, i, h), _rand_w(rng, i, h), _rand_w(rng, h, i)) for _ in range(e)]
    experts = [tuple(_qmat(m, asym) for m in trio) for trio in raw]
    x = _bf16_values(rng, t, h)
    L = rng.normal(size=(t, e))
    ids = router.select_topk(L, k)
    w = router.topk_weights(L, ids)
    got = ffn.moe_w4a16(x, lambda j: experts[j], ids, w)
    # brute force: decode the canonical bytes, evaluate every expert on every token
    dense = []
    for trio in raw:
        mats = []
        for m in trio:
            packed, sb, zp = quant.quantize_pack(m, asym)
            mats.append(_brute_dequant(packed, sb, zp, m.shape[0], m.shape[1], asym))
        dense.append(mats)
    for r in range(t):
        ys = [_brute_ffn(x[r].tolist(), *dense[j]) for j in range(e)]
        ref = [sum(w[r, c] * ys[ids[r, c]][n] for c in range(k)) for n in range(h)]
        assert np.allclose(got[r], ref, rtol=1e-10, atol=1e-13)


def test_slice_identity_and_dense_reduction():
    rng = np.random.default_rng(20)
    t, h, dense_i, e = 4, 256, 512, 4
    inter = dense_i // e
    G, U, D = _rand_w(rng, dense_i, h), _rand_w(rng, dense_i, h), _rand_w(rng, h, dense_i)
    x = _bf16_values(rng, t, h)
    dq = [_qmat(G, False), _qmat(U, False), _qmat(D, False)]
    dense = ffn.swiglu_w4a16(x, *dq)

    def sliced(j):
        sl = slice(j * inter, (j + 1) * inter)
        return _qmat(G[sl], False), _qmat(U[sl], False), _qmat(D[:, sl], False)

    # quantise(dense) sliced == quantise(slices), bit for bit (groups align with slices)
    for j in range(e):
        sl = slice(j * inter, (j + 1) * inter)
        gs, us, ds = sliced(j)
        assert np.array_equal(gs[0], dq[0][0][sl]) and np.array_equal(gs[1], dq[0][1][sl])
        assert np.array_equal(ds[0], dq[2][0][:, sl]) and np.array_equal(ds[1], dq[2][1][:, j:j + 1])
    ids = np.tile(np.arange(e), (t, 1))
    moe = ffn.moe_w4a16(x, sliced, ids, np.ones((t, e)))
    assert np.allclose(moe, dense, rtol=1e-12, atol=1e-14)
    # E = 1, k = 1, weight 1 is the dense FFN
    one = ffn.moe_w4a16(x, lambda j: dq, np.zeros((t, 1), np.int32), np.ones((t, 1)))
    assert np.array_equal(one, dense)


def test_zero_input_gives_zero_output():
    rng = np.random.default_rng(21)
    trio = tuple(_qmat(_rand_w(rng, *s), False) for s in ((128, 128), (128, 128), (128, 128)))
    x = np.zeros((3, 128), dtype=np.float32)
    assert np.all(ffn.moe_w4a16(x, lambda j: trio, np.zeros((3, 1), np.int32), np.ones((3, 1)), shared=trio) == 0)
    assert np.all(ffn.moe_w4a8(x, lambda j: trio, np.zeros((3, 1), np.int32), np.ones((3, 1)), shared=trio) == 0)


def test_shared_expert_adds_with_unit_weight():
    rng = np.random.default_rng(22)
    mk = lambda: tuple(_qmat(_rand_w(rng, *s), False) for s in ((128, 128), (128, 128), (128, 128)))
    routed, shared = mk(), mk()
    x = _bf16_values(rng, 3, 128)
    ids = np.zeros((3, 1), np.int32)
    base = ffn.moe_w4a16(x, lambda j: routed, ids, np.full((3, 1), 0.5))
    both = ffn.moe_w4a16(x, lambda j: routed, ids, np.full((3, 1), 0.5), shared=shared)
    assert np.allclose(both - base, ffn.swiglu_w4a16(x, *shared), rtol=1e-12, atol=1e-15)


def test_act_quant_worked_example_by_hand():
    # amax 127 -> scale exactly 1; half-way values go to the even neighbour
    row = np.array([[127.0, -63.5, 0.5, 1.5, 2.5, -0.5, 0.0, 3.25]], dtype=np.float32)
    q, s = ffn.act_quant_int8(row)
    assert s.tolist() == [1.0]
    assert q[0].tolist() == [127, -64, 0, 2, 2, 0, 0, 3]
    q0, s0 = ffn.act_quant_int8(np.zeros((1, 8), np.float32))
    assert s0.tolist() == [0.0] and np.all(q0 == 0)


def test_act_quant_invariants():
    rng = np.random.default_rng(23)
    a = rng.normal(0, 1, size=(200, 512)).astype(np.float32)
    a[:, :5] *= 10
    q, s = ffn.act_quant_int8(a)
    assert np.all(np.max(np.abs(q.astype(np.int64)), axis=1) == 127)
    # error bound: half a step, plus the float32 division slack
    err = np.abs(a.astype(np.float64) - q.astype(np.float64) * s.astype(np.float64)[:, None])
    assert np.all(err <= s.astype(np.float64)[:, None] * (0.5 + 2.0 ** -16))


@pytest.mark.parametrize("asym", [False, True])
def test_group_acc_bruteforce_and_bound(asym):
    rng = np.random.default_rng(24)
    t, n, k = 3, 5, 256
    qx = rng.integers(-128, 128, size=(t, k))
    qx[0] = -128
    m = _qmat(_rand_w(rng, n, k), asym)
    w8 = ffn.widen_int8(m)
    acc = ffn.group_acc(qx, w8)
    for a in range(t):
        for b in range(n):
            for g in range(2):
                ref = 0
                for c in range(128 * g, 128 * g + 128):
                    code = int(m[0][b, c]) - (int(m[2][b, g]) if asym else 0)
                    ref += int(qx[a, c]) * code
                assert acc[a, b, g] == ref
    bound = 128 * 128 * (15 if asym else 8)
    assert np.all(np.abs(acc) <= bound) and bound < 2 ** 31


def test_w4a8_equals_w4a16_when_activation_scale_is_one():
    rng = np.random.default_rng(25)
    t, h, i = 4, 256, 128
    x = rng.integers(-127, 128, size=(t, h)).astype(np.float32)
    x[:, 0] = 127.0                                  # amax 127 -> s_x = 1, q_x = x
    gate = _qmat(_rand_w(rng, i, h), False)
    qx, sx = ffn.act_quant_int8(x)
    assert np.all(sx == 1.0) and np.array_equal(qx.astype(np.float32), x)
    a8 = ffn.linear_w4a8(qx, sx, gate)
    a16 = ffn.linear_w4a16(x, gate)
    assert np.allclose(a8, a16, rtol=1e-12, atol=1e-12)


def test_w4a8_moe_close_to_w4a16_moe():
    """The two modes differ only by the INT8 activation rounding (a few per cent)."""
    rng = np.random.default_rng(26)
    t, h, i, e, k = 6, 256, 128, 4, 2
    experts = [tuple(_qmat(_rand_w(rng, *s), False) for s in ((i, h), (i, h), (h, i))) for _ in range(e)]
    x = _bf16_values(rng, t, h)
    L = rng.normal(size=(t, e))
    ids = router.select_topk(L, k)
    w = router.topk_weights(L, ids)
    a16 = ffn.moe_w4a16(x, lambda j: experts[j], ids, w)
    a8 = ffn.moe_w4a8(x, lambda j: experts[j], ids, w)
    assert 0 < ffn.max_rel_l2(a8, a16) < 0.05


def test_max_rel_l2_definition():
    ref = np.array([[3.0, 4.0], [0.0, 0.0]])
    assert ffn.max_rel_l2(np.array([[3.0, 4.5], [0.0, 0.0]]), ref) == pytest.approx(0.1)
    assert ffn.max_rel_l2(np.array([[3.0, 4.0], [0.0, 1e-30]]), ref) == np.inf
