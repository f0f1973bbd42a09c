"""Pins of the oracle's INT4 g128 quantiser and packer against what the pages and
the arithmetic fix (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _weights(n, k, seed, outliers=True):
    rng = np.random.default_rng(seed)
    w = rng.normal(0.0, 0.02, size=(n, k)).astype(np.float32)
    if outliers:
        pos = rng.choice(n * k, max(1, n * k // 1000), replace=False)
        w.reshape(-1)[pos] *= 20
    # a few groups with very different magnitudes, one all-zero group
    w[0, :128] *= 1e-3
    w[1, 128:256] *= 1e3
    w[2, :128] = 0.0
    return w


@pytest.mark.parametrize("seed", [0, 1])
def test_sym_codes_are_nearest_by_brute_force(seed):
    w = _weights(64, 512, seed)
    q, s = quant.quantize_sym(w)
    s64 = np.repeat(s.astype(np.float64), 128, axis=1)
    nz = s64 > 0
    r = w.astype(np.float64)[nz] / s64[nz]
    codes = np.arange(-8, 8, dtype=np.float64)
    best = np.min(np.abs(r[:, None] - codes[None, :]), axis=1)
    chosen = np.abs(r - q[nz])
    # the fp32 division may move a value across a rounding boundary by ~2^-21
    assert np.all(chosen <= best + 1e-6)
    assert np.all(q[~nz] == 0)


@pytest.mark.parametrize("seed", [0, 1])
def test_sym_half_step_bound(seed):
    w = _weights(64, 1024, seed)
    q, s = quant.quantize_sym(w)
    what = quant.dequantize(q, s)
    s64 = np.repeat(s.astype(np.float64), 128, axis=1)
    assert np.all(np.abs(w.astype(np.float64) - what) <= s64 / 2 * (1 + 2.0 ** -20))


def test_sym_scale_is_nearest_binary16_of_amax_over_7():
    w = _weights(32, 512, 7)
    _, s = quant.quantize_sym(w)
    amax = np.max(np.abs(w.reshape(32, 4, 128)), axis=2).astype(np.float32)
    t = (amax / np.float32(7)).astype(np.float64)     # the fp32 quotient, exactly
    s64 = s.astype(np.float64)
    lo = np.nextafter(s, np.float16(-np.inf)).astype(np.float64)
    hi = np.nextafter(s, np.float16(np.inf)).astype(np.float64)
    assert np.all(np.abs(s64 - t) <= np.abs(lo - t))
    assert np.all(np.abs(s64 - t) <= np.abs(hi - t))


def test_sym_every_group_reaches_plus_minus_7():
    w = _weights(64, 1024, 3)
    q, s = quant.quantize_sym(w)
    normal = (s.astype(np.float32) >= np.float32(2.0 ** -14))
    qmax = np.max(np.abs(q.reshape(64, 8, 128).astype(np.int64)), axis=2)
    assert np.all(qmax[normal] == 7)
    assert np.all(q >= -8) and np.all(q <= 7)


def test_sym_exact_ties_round_half_to_even():
    # group amax = 7 * 2^-6 makes the scale exactly 2^-6; (m + 1/2) * 2^-6 is an exact tie
    s0 = 2.0 ** -6
    m = np.arange(-7, 7)
    row = np.zeros(128, dtype=np.float32)
    row[0] = 7 * s0
    row[1:1 + m.size] = ((m + 0.5) * s0).astype(np.float32)
    q, s = quant.quantize_sym(row[None, :])
    assert s[0, 0] == np.float16(s0)
    # expected: the even neighbour of m + 1/2, worked out by hand
    expect = np.array([mm if mm % 2 == 0 else mm + 1 for mm in m])
    assert np.array_equal(q[0, 1:1 + m.size], expect)
    assert q[0, 0] == 7


def test_sym_zero_and_tiny_groups():
    w = np.zeros((2, 256), dtype=np.float32)
    w[1, :128] = 1e-12          # a / 7 underflows binary16 -> scale 0, codes 0
    q, s = quant.quantize_sym(w)
    assert np.all(s.astype(np.float32) == 0) and np.all(q == 0)


def test_sym_rejects_bad_input():
    with pytest.raises(ValueError):
        quant.quantize_sym(np.zeros((2, 100), dtype=np.float32))
    with pytest.raises(ValueError):
        quant.quantize_sym(np.full((1, 128), np.inf, dtype=np.float32))
    with pytest.raises(ValueError):
        quant.quantize_sym(np.full((1, 128), 1e6, dtype=np.float32))    # scale > 65504


def test_f16_round_up_definition():
    rng = np.random.default_rng(5)
    t = np.concatenate([rng.uniform(0, 1, 5000), rng.uniform(0, 1e-5, 2000),
                        np.array([0.0, 1.0, 0.5, 2.0 ** -24, 65504.0])]).astype(np.float32)
    h = quant.f32_to_f16_up(t)
    h64 = h.astype(np.float64)
    below = np.nextafter(h, np.float16(-np.inf)).astype(np.float64)
    assert np.all(h64 >= t.astype(np.float64))
    assert np.all((below < t.astype(np.float64)) | (h64 == 0))


@pytest.mark.parametrize("seed", [0, 1])
def test_asym_codes_are_nearest_by_brute_force(seed):
    w = _weights(64, 512, seed)
    w[3] = np.abs(w[3])                    # an all-positive row
    w[4] = -np.abs(w[4])                   # an all-negative row
    q, s, z = quant.quantize_asym(w)
    s64 = np.repeat(s.astype(np.float64), 128, axis=1)
    z64 = np.repeat(z.astype(np.float64), 128, axis=1)
    nz = s64 > 0
    r = w.astype(np.float64)[nz] / s64[nz]
    cand = np.arange(16, dtype=np.float64)[None, :] - z64[nz][:, None]
    best = np.min(np.abs(r[:, None] - cand), axis=1)
    chosen = np.abs(r - (q[nz] - z64[nz]))
    assert np.all(chosen <= best + 1e-6)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_asym_half_step_bound_and_min_code(seed):
    w = _weights(128, 1024, seed)
    q, s, z = quant.quantize_asym(w)
    what = quant.dequantize(q, s, z)
    s64 = np.repeat(s.astype(np.float64), 128, axis=1)
    assert np.all(np.abs(w.astype(np.float64) - what) <= s64 / 2 * (1 + 2.0 ** -19))
    assert np.all(z <= 15) and np.all(q <= 15)
    # the group minimum (when negative) maps to code 0
    wg = w.reshape(128, 8, 128)
    qg = q.reshape(128, 8, 128)
    amin = np.argmin(wg, axis=2)
    neg = np.min(wg, axis=2) < 0
    codes_at_min = np.take_along_axis(qg, amin[..., None], axis=2)[..., 0]
    assert np.all(codes_at_min[neg & (s.astype(np.float32) > 0)] == 0)


def test_nibble_pack_exhaustive_roundtrip():
    lo, hi = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    codes = np.stack([lo.ravel(), hi.ravel()], axis=1)              # 256 (lo, hi) pairs
    packed = quant.pack_nibbles(codes)
    assert np.array_equal(packed[:, 0], (lo.ravel() | (hi.ravel() << 4)).astype(np.uint8))
    assert np.array_equal(np.sort(packed[:, 0]), np.arange(256, dtype=np.uint8))
    assert np.array_equal(quant.unpack_nibbles(packed, 2, signed=False), codes)
    signed = np.where(codes >= 8, codes - 16, codes)
    assert np.array_equal(quant.pack_nibbles(signed), packed)
    assert np.array_equal(quant.unpack_nibbles(packed, 2, signed=True), signed)


def test_pack_low_nibble_first_by_hand():
    assert quant.pack_nibbles(np.array([[1, 2, -1, 7]]))[0].tolist() == [0x21, 0x7F]
    # odd count along g (zero points): pad nibble is 0
    assert quant.pack_nibbles(np.array([[5, 6, 9]]))[0].tolist() == [0x65, 0x09]


def test_canonical_roundtrip():
    w = _weights(32, 384, 11)
    for asym in (False, True):
        packed, sb, zp = quant.quantize_pack(w, asym)
        q, s, z = quant.unpack_canonical(packed, sb, zp, 384, asym)
        ref = quant.quantize_asym(w) if asym else quant.quantize_sym(w)
        assert np.array_equal(q, ref[0].astype(np.int64))
        assert np.array_equal(s.view(np.uint16), ref[1].view(np.uint16))
        if asym:
            assert np.array_equal(z, ref[2].astype(np.int64))
        assert packed.nbytes + sb.nbytes + (zp.nbytes if asym else 0) == quant.packed_bytes(32, 384, asym)


def test_packed_size_about_a_quarter_of_fp16():
    with open(os.path.join(GOLDEN, "size_claims.json")) as f:
        claims = json.load(f)
    # nibbles alone: exactly a quarter of fp16 (the pages' 14 GB -> 3.5 GB for 7e9 weights)
    p = claims["params_7b"]
    assert p * 2 / 1e9 == pytest.approx(claims["fp16_gb_7b"], rel=0.01)
    assert p / 2 / 1e9 == pytest.approx(claims["int4_gb_7b"], rel=0.01)
    # the g128 format adds one fp16 scale per 128 weights (and a 4-bit zero point)
    for asym, ratio in ((False, 0.2578125), (True, 0.259765625)):
        r = quant.packed_bytes(4096, 4096, asym) / (4096 * 4096 * 2)
        assert r == pytest.approx(ratio, abs=1e-9)
        assert claims["quarter_lo"] <= r <= claims["quarter_hi"]
