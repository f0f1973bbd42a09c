"""Device tile layout of one INT4 g128 matrix (oracle re-derivation of the spec).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

The pages fix the canonical format (nibbles, per-group scales, optional zero
points); the device layout is this library's own fixed permutation of those
bytes, written out here from its specification and nothing else:

Columns.  A matrix has N output columns (rows of the weight) and K reduction
elements.  ``plain`` keeps column order.  ``gate_up`` takes a stacked
[gate; up] matrix of 2I rows and interleaves 16-column blocks: device block
2b holds gate rows [16b, 16b+16), device block 2b+1 holds up rows
[I+16b, I+16b+16).

Codes.  Every nibble holds an unsigned value d: d = q + 8 for the symmetric
format (implied zero point 8), d = q for the asymmetric one.

Weights.  One 1024-byte tile per (column block cb, group g), tiles ordered
cb-major: byte offset 1024 * (cb * G + g).  Inside a tile, lane L in [0, 64)
owns bytes [16 L, 16 L + 16): column c = L % 16 of the block and quarter
kq = L // 16.  Its little-endian 32-bit word s in [0, 4) holds the elements
k = 128 g + 32 s + 8 kq + e, e in [0, 8), element e at nibble position
p(e) = [0, 2, 4, 6, 1, 3, 5, 7][e] (bits 4p .. 4p+3): byte j of the word holds
element j in its low nibble and element j + 4 in its high nibble.

Scales.  Binary16 bits, [N/16][G][16][SG] (same column order; a column's SG entries
of one tile are adjacent), starting at byte align256(N K / 2).  SG is the number of
scale groups per 128-element tile: 1 for
the default group of 128, 128 / group for groups of 32 or 64 (entry j of tile g is
the scale of k in [128 g + j 128/SG, 128 g + (j + 1) 128/SG)), and 1 for groups of
256, where each tile carries the scale of the 256-group it lies in (both tiles of a
group hold the same value).  In general entry (tile g, j) holds canonical group
(128 g + j 128/SG) // group.

Zeros (asymmetric only; groups of 128 or 256).  One byte z per (column, tile),
[N/16][G][16] (the zero point of the tile's group), starting after the scales at
align256(.) of their end.

Total size: align256(N K/2) + align256(2 N G SG) (+ align256(N G)), G = K / 128.

Pinned by (tests/test_oracle_layout.py): unpack(layout(x)) == x on random
canonical inputs (both column orders, both formats), and a hand-computed
single-element placement.
"""
import numpy as np

from .quant import GROUP, GROUPS, unpack_canonical, unpack_crumbs

NIBBLE_POS = np.array([0, 2, 4, 6, 1, 3, 5, 7])


def _a256(x):
    return (x + 255) // 256 * 256


def sub_groups(group):
    """Scale groups per 128-element tile."""
    return 128 // group if group < 128 else 1


def device_bytes(n, k, asymmetric, group=GROUP):
    g = k // GROUP
    total = _a256(n * k // 2) + _a256(2 * n * g * sub_groups(group))
    if asymmetric:
        total += _a256(n * g)
    return total


def column_source(n, gate_up):
    """Device column j -> source row of the canonical matrix."""
    j = np.arange(n)
    if not gate_up:
        return j
    half = n // 2
    cb, c = j // 16, j % 16
    return np.where(cb % 2 == 0, 16 * (cb // 2) + c, half + 16 * (cb // 2) + c)


def _scale_source(k, group):
    """Canonical group index of each device scale entry (tile g, j), shape [G, SG]."""
    sg = sub_groups(group)
    g = np.arange(k // GROUP)[:, None]
    j = np.arange(sg)[None, :]
    return (GROUP * g + j * (GROUP // sg)) // group


def to_device(packed, scale_bits, zeros_packed, n, k, asymmetric, gate_up, group=GROUP):
    """Canonical bytes -> device bytes (uint8 array of device_bytes(n, k, asym, group))."""
    if n % (32 if gate_up else 16) or k % GROUP or k % group or group not in GROUPS:
        raise ValueError("shape not supported by the device layout")
    if asymmetric and group < GROUP:
        raise ValueError("zero points need groups of 128 or 256")
    g = k // GROUP
    sg = sub_groups(group)
    q, s, z = unpack_canonical(packed, scale_bits, zeros_packed, k, asymmetric, group)
    d = q + 8 if not asymmetric else q                       # unsigned nibble values
    src = column_source(n, gate_up)
    d = d[src]
    s = s[src]
    out = np.zeros(device_bytes(n, k, asymmetric, group), dtype=np.uint8)
    # weights: element (col j, k) -> tile (j//16, k//128), lane, word, nibble
    words = np.zeros(n * k // 8, dtype=np.uint64)
    jj, kk = np.meshgrid(np.arange(n), np.arange(k), indexing="ij")
    cb, c = jj // 16, jj % 16
    gg, r = kk // GROUP, kk % GROUP
    sidx, rem = r // 32, r % 32
    kq, e = rem // 8, rem % 8
    lane = kq * 16 + c
    word_index = ((cb * g + gg) * 1024 + lane * 16 + sidx * 4) // 4
    shift = 4 * NIBBLE_POS[e]
    np.add.at(words, word_index.ravel(), (d.astype(np.uint64) << shift.astype(np.uint64)).ravel())
    out[: n * k // 2] = words.astype("<u4").view(np.uint8)
    # scales [N/16][G][16][SG]: entry (tile, j) of a column from its canonical group
    so = _a256(n * k // 2)
    srcg = _scale_source(k, group)                                    # [G, SG]
    se = s.view(np.uint16)[:, srcg]                                   # [N, G, SG]
    sc = se.reshape(n // 16, 16, g, sg).transpose(0, 2, 1, 3).reshape(-1)
    out[so: so + 2 * n * g * sg] = sc.astype("<u2").view(np.uint8)
    if asymmetric:
        zo = so + _a256(2 * n * g * sg)
        ze = z[src][:, srcg[:, 0]]                                    # [N, G]
        zz = ze.reshape(n // 16, 16, g).transpose(0, 2, 1).reshape(-1)
        out[zo: zo + n * g] = zz.astype(np.uint8)
    return out


def from_device(dev, n, k, asymmetric, gate_up, group=GROUP):
    """Device bytes -> (q int64 [N, K], scale bits uint16 [N, K/group], zeros int64
    [N, K/group] or None), in canonical row order (for groups of 256 the scale and zero
    point are read from the first tile of each group)."""
    g = k // GROUP
    sg = sub_groups(group)
    dev = np.asarray(dev, dtype=np.uint8)
    words = dev[: n * k // 2].view("<u4").astype(np.int64)
    jj, kk = np.meshgrid(np.arange(n), np.arange(k), indexing="ij")
    cb, c = jj // 16, jj % 16
    gg, r = kk // GROUP, kk % GROUP
    sidx, rem = r // 32, r % 32
    kq, e = rem // 8, rem % 8
    lane = kq * 16 + c
    word_index = ((cb * g + gg) * 1024 + lane * 16 + sidx * 4) // 4
    d = (words[word_index] >> (4 * NIBBLE_POS[e])) & 0xF
    so = _a256(n * k // 2)
    sc = dev[so: so + 2 * n * g * sg].view("<u2").reshape(n // 16, g, 16, sg).transpose(0, 2, 1, 3)
    sc = sc.reshape(n, g * sg)
    if group > GROUP:
        sc = sc[:, :: group // GROUP]
    zz = None
    if asymmetric:
        zo = so + _a256(2 * n * g * sg)
        zz = dev[zo: zo + n * g].reshape(n // 16, g, 16).transpose(0, 2, 1).reshape(n, g).astype(np.int64)
        if group > GROUP:
            zz = zz[:, :: group // GROUP]
    q = d if asymmetric else d - 8
    src = column_source(n, gate_up)
    inv = np.empty_like(src)
    inv[src] = np.arange(n)
    return q[inv], sc[inv].astype(np.uint16), (zz[inv] if zz is not None else None)


# ---------------------------------------------------------------- 8-bit weights
# INT8 device layout (W8A8): one 2048-byte tile per (16-column block cb, group g),
# tiles cb-major at byte 2048 * (cb * G + g).  The tile is two 1024-byte halves,
# half i for k in [128 g + 64 i, 128 g + 64 i + 64); inside a half, lane L in [0, 64)
# (column c = L % 16, quarter kq = L // 16) owns 16 bytes: bytes 0..7 are
# k = 128 g + 64 i + 8 kq + e and bytes 8..15 are k = 128 g + 64 i + 32 + 8 kq + e,
# e in [0, 8), as two's-complement int8 codes.  Scales as for INT4, binary16
# [N/16][G][16] at byte align256(N K).  Same column orders (plain / gate-up).

def device_bytes8(n, k):
    return _a256(n * k) + _a256(2 * n * (k // GROUP))


def _offsets8(n, k):
    g = k // GROUP
    jj, kk = np.meshgrid(np.arange(n), np.arange(k), indexing="ij")
    cb, c = jj // 16, jj % 16
    gg, r = kk // GROUP, kk % GROUP
    half, rr = r // 64, r % 64
    hi, kq, e = rr // 32, (rr % 32) // 8, rr % 8
    lane = kq * 16 + c
    return (cb * g + gg) * 2048 + half * 1024 + lane * 16 + hi * 8 + e


def to_device8(q, scale_bits, n, k, gate_up):
    """INT8 codes [N, K] + scale bits [N, G] -> device bytes (device_bytes8(n, k))."""
    if n % (32 if gate_up else 16) or k % GROUP:
        raise ValueError("shape not supported by the device layout")
    g = k // GROUP
    src = column_source(n, gate_up)
    qd = np.asarray(q, dtype=np.int64)[src]
    s = np.asarray(scale_bits, dtype=np.uint16)[src]
    out = np.zeros(device_bytes8(n, k), dtype=np.uint8)
    out[_offsets8(n, k).ravel()] = (qd & 0xFF).astype(np.uint8).ravel()
    so = _a256(n * k)
    sc = s.reshape(n // 16, 16, g).transpose(0, 2, 1).reshape(-1)
    out[so: so + 2 * n * g] = sc.astype("<u2").view(np.uint8)
    return out


def from_device8(dev, n, k, gate_up):
    """Device bytes -> (q int64 [N, K], scale bits uint16 [N, G]) in canonical row order."""
    g = k // GROUP
    dev = np.asarray(dev, dtype=np.uint8)
    q = dev[_offsets8(n, k)].view(np.int8).astype(np.int64)
    so = _a256(n * k)
    sc = dev[so: so + 2 * n * g].view("<u2").reshape(n // 16, g, 16).transpose(0, 2, 1).reshape(n, g)
    src = column_source(n, gate_up)
    inv = np.empty_like(src)
    inv[src] = np.arange(n)
    return q[inv], sc[inv].astype(np.uint16)


# ---------------------------------------------------------------- 2-bit weights
# INT2 device layout (cold experts): one 512-byte tile per (16-column block cb, group g),
# tiles cb-major at byte 512 * (cb * G + g).  Lane L in [0, 64) (column c = L % 16,
# quarter kq = L // 16) owns bytes [8 L, 8 L + 8): two little-endian 32-bit words.  The
# element k = 128 g + 32 s + 8 kq + e (K step s in [0, 4), e in [0, 8)) is in word s // 2,
# byte m = e % 4 of that word, bit field f = 2 (s % 2) + e // 4 (bits 8 m + 2 f and
# 8 m + 2 f + 1), as the unsigned value d = q + 2.  (One shift-and-mask then gives the
# four elements of a field as bytes, for the INT8 operand; one shift-mask-or gives two
# of them, four apart in k -- bytes m and m + 2 -- as a bf16 pair under a constant
# exponent, for the bf16 operand.)  Scales as for INT4, binary16 [N/16][G][16] at byte
# align256(N K / 4).  Same column orders (plain / gate-up).

def device_bytes2(n, k):
    return _a256(n * k // 4) + _a256(2 * n * (k // GROUP))


def _offsets2(n, k):
    """(byte offset, bit shift) of every element (column j, k) in device order."""
    g = k // GROUP
    jj, kk = np.meshgrid(np.arange(n), np.arange(k), indexing="ij")
    cb, c = jj // 16, jj % 16
    gg, r = kk // GROUP, kk % GROUP
    s, rem = r // 32, r % 32
    kq, e = rem // 8, rem % 8
    lane = kq * 16 + c
    word = s // 2
    m, f = e % 4, 2 * (s % 2) + e // 4
    byte = (cb * g + gg) * 512 + lane * 8 + word * 4 + m
    return byte, 2 * f


def to_device2(packed, scale_bits, n, k, gate_up):
    """Canonical 2-bit bytes [N, K/4] + scale bits [N, G] -> device bytes
    (device_bytes2(n, k))."""
    if n % (32 if gate_up else 16) or k % GROUP:
        raise ValueError("shape not supported by the device layout")
    g = k // GROUP
    q = unpack_crumbs(packed, k)
    src = column_source(n, gate_up)
    d = (q[src] + 2).astype(np.int64)
    s = np.asarray(scale_bits, dtype=np.uint16)[src]
    out = np.zeros(device_bytes2(n, k), dtype=np.uint8)
    byte, shift = _offsets2(n, k)
    acc = np.zeros(n * k // 4, dtype=np.int64)
    np.add.at(acc, byte.ravel(), (d << shift).ravel())
    out[: n * k // 4] = acc.astype(np.uint8)
    so = _a256(n * k // 4)
    sc = s.reshape(n // 16, 16, g).transpose(0, 2, 1).reshape(-1)
    out[so: so + 2 * n * g] = sc.astype("<u2").view(np.uint8)
    return out


def from_device2(dev, n, k, gate_up):
    """Device bytes -> (q int64 [N, K] in [-2, 1], scale bits uint16 [N, G]) in canonical
    row order."""
    g = k // GROUP
    dev = np.asarray(dev, dtype=np.uint8).astype(np.int64)
    byte, shift = _offsets2(n, k)
    q = ((dev[byte] >> shift) & 0x3) - 2
    so = _a256(n * k // 4)
    sc = np.asarray(dev[so: so + 2 * n * g], dtype=np.uint8).view("<u2")
    sc = sc.reshape(n // 16, g, 16).transpose(0, 2, 1).reshape(n, g)
    src = column_source(n, gate_up)
    inv = np.empty_like(src)
    inv[src] = np.arange(n)
    return q[inv], sc[inv].astype(np.uint16)
