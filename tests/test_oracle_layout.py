"""Pins of the oracle's device-layout re-derivation (CPU only)."""
import numpy as np
import pytest

from oracle import layout, quant


@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("gate_up", [False, True])
def test_roundtrip(asym, gate_up):
    rng = np.random.default_rng(7)
    n, k = 64, 384
    w = rng.normal(0, 0.02, size=(n, k)).astype(np.float32)
    packed, sb, zp = quant.quantize_pack(w, asym)
    dev = layout.to_device(packed, sb, zp, n, k, asym, gate_up)
    assert dev.size == layout.device_bytes(n, k, asym)
    q, s, z = layout.from_device(dev, n, k, asym, gate_up)
    q0, s0, z0 = quant.unpack_canonical(packed, sb, zp, k, asym)
    assert np.array_equal(q, q0)
    assert np.array_equal(s, s0.view(np.uint16))
    if asym:
        assert np.array_equal(z, z0)


def test_single_element_placement_by_hand():
    # one non-zero code: row 17 (block 1, column 1), k = 128 + 32*2 + 8*3 + 5
    # -> tile (1, 1) of a 2-group matrix = tile index 3, lane 3*16 + 1 = 49, word 2,
    #    element 5 at nibble position 3 (byte 1, high nibble)
    n, k = 32, 256
    q = np.zeros((n, k), dtype=np.int64)
    kk = 128 + 64 + 24 + 5
    q[17, kk] = 3                                     # symmetric code 3 -> nibble value 11
    packed = quant.pack_nibbles(q)
    sb = np.full((n, 2), np.float16(1.0).view(np.uint16), dtype=np.uint16)
    dev = layout.to_device(packed, sb, None, n, k, False, False)
    word = dev[3 * 1024 + 49 * 16 + 2 * 4: 3 * 1024 + 49 * 16 + 3 * 4].view("<u4")[0]
    assert (int(word) >> 12) & 0xF == 11
    # every other nibble of the weights holds 8 (code 0)
    w = dev[: n * k // 2].view("<u4").astype(np.int64)
    nib = np.stack([(w >> (4 * p)) & 0xF for p in range(8)], axis=1)
    assert np.count_nonzero(nib != 8) == 1
    # scales: [N/16][G][16] -> row 17 group 1 at index (1*2 + 1)*16 + 1
    so = n * k // 2
    sc = dev[so: so + 2 * n * 2].view("<u2")
    assert sc[(1 * 2 + 1) * 16 + 1] == np.float16(1.0).view(np.uint16)


def test_gate_up_interleave_by_hand():
    src = layout.column_source(64, True)
    assert src[:16].tolist() == list(range(16))           # gate rows 0..15
    assert src[16:32].tolist() == list(range(32, 48))     # up rows 0..15 (I = 32)
    assert src[32:48].tolist() == list(range(16, 32))
    assert src[48:64].tolist() == list(range(48, 64))
