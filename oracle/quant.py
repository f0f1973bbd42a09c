"""INT4 group-128 weight quantisation and nibble packing (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Format (page "从FP32到INT4：大语言模型量化压缩实战指南", §1.3 分组量化技术解析:
groups of 128 along the reduction dimension K, each group with its own scale
from its own min/max, a zero point only in the asymmetric variant; page
"高效大语言模型推理实践：INT4量化与MoE架构的融合探索", 核心实现细节 / INT4量化实现:
4-bit integers plus an independent scale per group):

* weight ``w`` of shape [N, K], K a multiple of 128, group g covers
  k in [128 g, 128 g + 128) of every row;
* one binary16 scale per (row, group), and in the asymmetric variant one
  unsigned 4-bit zero point per (row, group);
* two 4-bit codes per byte, the even k in the low nibble.

Readings where the pages leave a step open (each listed in the design doc):

* symmetric scale = amax / 7 computed as an IEEE float32 division, then
  rounded to nearest-even binary16; codes are rint(w / s) with the *stored*
  scale, clamped to [-8, 7], stored as two's-complement nibbles;
* asymmetric range [min(min w, 0), max(max w, 0)], scale = (mx - mn) / 15 in
  float32 rounded *upward* to binary16 (so the half-step bound holds at the
  group maximum), z = clamp(rint(-mn / s), 0, 15),
  q = clamp(rint(w / s) + z, 0, 15);
* a group whose scale is zero gets s = 0, codes 0 (and z = 0).

Other group sizes (page "MoE推理优化实战：4bit存储+INT8计算的W4A8路线解析", §5.3:
group sizes 32 / 64 / 128 / 256 chosen per expert by how often it is hit): the same
definitions with groups of ``group`` elements along K (K a multiple of it); the
scale tables then have K / group columns.  The group of a quantised matrix is implied
by its shapes (K / number of scale columns).

2-bit codes for cold experts (quantize_sym2, pack_crumbs): see quantize_sym2.

Pinned by (tests/test_oracle_quant.py, tests/test_oracle_groups.py, tests/test_oracle_int2.py):
brute-force nearest-code search over
all 16 codes for every element, the half-step error bound, constructed exact
ties (half-to-even), the +-7 / code-0 invariants, exhaustive nibble
round-trip of all 256 bytes, and the packed-size formula against the "about
a quarter of fp16" statement.
"""
import numpy as np

GROUP = 128
GROUPS = (32, 64, 128, 256)


def _groups(w, group=GROUP):
    w32 = np.asarray(w, dtype=np.float32)
    if w32.ndim != 2:
        raise ValueError("weight must be 2-D [N, K]")
    if group not in GROUPS:
        raise ValueError("group must be 32, 64, 128 or 256")
    n, k = w32.shape
    if k % group != 0:
        raise ValueError(f"K must be a multiple of {group}")
    if not np.all(np.isfinite(w32)):
        raise ValueError("non-finite weight")
    return w32.reshape(n, k // group, group)


def group_of(k, scales):
    """Group size implied by a matrix of K columns and its scale table."""
    return k // np.asarray(scales).shape[1]


def f32_to_f16_up(t):
    """Round non-negative float32 values up (toward +inf) to binary16.

    Definition: the smallest binary16 value that is >= t.  Built from the
    library's round-to-nearest-even conversion plus one step of nextafter.
    """
    t = np.asarray(t, dtype=np.float32)
    h = t.astype(np.float16)
    low = h.astype(np.float32) < t
    h = h.copy()
    h[low] = np.nextafter(h[low], np.float16(np.inf))
    return h


def quantize_sym(w, group=GROUP):
    """Symmetric INT4 quantisation (groups of ``group`` along K, 128 by default).

    Returns (q int8 [N, K] in [-8, 7], scales float16 [N, K/group]).
    Follows §1.3 of the FP32->INT4 guide (per-group scale, no zero point for
    the symmetric variant) with the amax / 7 reading of the scale.
    """
    wg = _groups(w, group)
    amax = np.max(np.abs(wg), axis=2)                       # exact in fp32
    s16 = (amax / np.float32(7.0)).astype(np.float16)       # fp32 divide, RNE to fp16
    if not np.all(np.isfinite(s16)):
        raise ValueError("scale overflows binary16")
    s32 = s16.astype(np.float32)
    q = np.zeros(wg.shape, dtype=np.float32)
    nz = s32 > 0
    # fp32 division by the stored scale, then round-half-to-even
    q[nz] = np.rint(wg[nz] / s32[nz][:, None])
    q = np.clip(q, -8, 7)
    return q.reshape(np.asarray(w).shape).astype(np.int8), s16


def quantize_asym(w, group=GROUP):
    """Asymmetric INT4 quantisation with an unsigned 4-bit zero point.

    Returns (q uint8 [N, K] in [0, 15], scales float16 [N, G], zeros uint8 [N, G]).
    Follows §1.3 of the FP32->INT4 guide (each group computes its own min/max,
    the asymmetric variant stores a zero point).
    """
    wg = _groups(w, group)
    mn = np.minimum(np.min(wg, axis=2), np.float32(0))
    mx = np.maximum(np.max(wg, axis=2), np.float32(0))
    t = (mx - mn) / np.float32(15.0)                          # fp32 ops, RNE
    s16 = f32_to_f16_up(t)
    if not np.all(np.isfinite(s16)):
        raise ValueError("scale overflows binary16")
    s32 = s16.astype(np.float32)
    n, g, _ = wg.shape
    z = np.zeros((n, g), dtype=np.float32)
    q = np.zeros(wg.shape, dtype=np.float32)
    nz = s32 > 0
    z[nz] = np.clip(np.rint(-mn[nz] / s32[nz]), 0, 15)
    q[nz] = np.clip(np.rint(wg[nz] / s32[nz][:, None]) + z[nz][:, None], 0, 15)
    return (q.reshape(np.asarray(w).shape).astype(np.uint8), s16, z.astype(np.uint8))


def quantize_sym8(w):
    """Symmetric INT8 g128 quantisation: the W8A8 comparison format.

    Returns (q int8 [N, K] in [-127, 127], scales float16 [N, K/128]).  Page
    "MoE推理优化实战：4bit存储+INT8计算的W4A8路线解析" lists W8A8 (INT8 weights and
    INT8 compute) as the accuracy-safe route to try first; its weight format is not
    spelled out, so it takes the same per-group structure as the INT4 format: per
    group of 128, s = amax / 127 as an IEEE float32 division, rounded *upward* to
    binary16 (as for the asymmetric INT4 scale: with 127 levels a nearest-even
    binary16 scale -- subnormal for small groups -- can fall below amax / 127 by more
    than half a step, and the clamped group maximum would then miss the half-step
    bound), q = clamp(rint(w / s), -127, 127) with the stored scale; a zero scale
    gives codes 0.
    """
    wg = _groups(w)
    amax = np.max(np.abs(wg), axis=2)
    s16 = f32_to_f16_up(amax / np.float32(127.0))
    if not np.all(np.isfinite(s16)):
        raise ValueError("scale overflows binary16")
    s32 = s16.astype(np.float32)
    q = np.zeros(wg.shape, dtype=np.float32)
    nz = s32 > 0
    q[nz] = np.rint(wg[nz] / s32[nz][:, None])
    q = np.clip(q, -127, 127)
    return q.reshape(np.asarray(w).shape).astype(np.int8), s16


def quantize_sym2(w):
    """Symmetric INT2 g128 quantisation: the cold-expert format.

    Returns (q int8 [N, K] in [-2, 1], scales float16 [N, K/128]).  Page "大模型之
    Dense、MoE与量化", APEX section: experts get precision by importance, commonly
    used experts 4 bits and rarely used ("cold") experts 2 bits.  The page does not
    spell the 2-bit format out; it takes the INT4 format's structure with b = 2: per
    group of 128 along K, s = amax / (2^(b-1) - 1) = amax, q = clamp(rint(w / s), -2, 1)
    with the stored scale (IEEE fp32 division, half-to-even), two's-complement codes,
    four per byte.  The scale is amax rounded *upward* to binary16 (as for the 8-bit
    format): with a single positive level, a nearest-even scale below amax (subnormal
    for tiny groups) would clamp the group maximum past half a step.  So |w / s| <= 1
    and the codes are -1, 0 and 1 (-2, like -8 in INT4, is never produced); a zero
    scale gives codes 0.
    """
    wg = _groups(w)
    amax = np.max(np.abs(wg), axis=2)
    s16 = f32_to_f16_up(amax)
    if not np.all(np.isfinite(s16)):
        raise ValueError("scale overflows binary16")
    s32 = s16.astype(np.float32)
    q = np.zeros(wg.shape, dtype=np.float32)
    nz = s32 > 0
    q[nz] = np.rint(wg[nz] / s32[nz][:, None])
    q = np.clip(q, -2, 1)
    return q.reshape(np.asarray(w).shape).astype(np.int8), s16


def pack_crumbs(codes):
    """Four 2-bit codes per byte along the last axis, index 4 j + i in bits 2 i, 2 i + 1
    of byte j (two's complement, code & 3); a partial last byte is zero-padded."""
    c = np.asarray(codes).astype(np.int64) & 0x3
    pad = (-c.shape[-1]) % 4
    if pad:
        c = np.concatenate([c, np.zeros(c.shape[:-1] + (pad,), dtype=np.int64)], axis=-1)
    out = c[..., 0::4] | (c[..., 1::4] << 2) | (c[..., 2::4] << 4) | (c[..., 3::4] << 6)
    return out.astype(np.uint8)


def unpack_crumbs(packed, count):
    """Inverse of pack_crumbs: the first ``count`` signed codes along the last axis."""
    p = np.asarray(packed, dtype=np.int64)
    out = np.empty(p.shape[:-1] + (4 * p.shape[-1],), dtype=np.int64)
    for i in range(4):
        out[..., i::4] = (p >> (2 * i)) & 0x3
    out = out[..., :count]
    return np.where(out >= 2, out - 4, out)


def packed_bytes2(n, k):
    """Bytes of the canonical 2-bit format: N*K/4 code bytes + 2*N*(K/128) scale bytes."""
    return n * k // 4 + 2 * n * (k // GROUP)


def dequantize(q, scales, zeros=None):
    """w_hat = (q - z) * s in float64 (exact: a small integer times a binary16)."""
    q = np.asarray(q, dtype=np.int64)
    n, k = q.shape
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    z = np.zeros_like(s) if zeros is None else np.asarray(zeros, dtype=np.float64)
    group = group_of(k, s)
    qg = q.reshape(n, k // group, group).astype(np.float64)
    return ((qg - z[:, :, None]) * s[:, :, None]).reshape(n, k)


def pack_nibbles(codes):
    """Two 4-bit codes per byte along the last axis, the even index in the low nibble.

    Signed codes are stored as two's complement (code & 0xF).
    """
    c = np.asarray(codes).astype(np.int64) & 0xF
    if c.shape[-1] % 2:
        pad = np.zeros(c.shape[:-1] + (1,), dtype=np.int64)
        c = np.concatenate([c, pad], axis=-1)
    lo = c[..., 0::2]
    hi = c[..., 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed, count, signed):
    """Inverse of pack_nibbles: the first ``count`` codes along the last axis."""
    p = np.asarray(packed, dtype=np.int64)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int64)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = (p >> 4) & 0xF
    out = out[..., :count]
    if signed:
        out = np.where(out >= 8, out - 16, out)
    return out


def quantize_pack(w, asymmetric, group=GROUP):
    """Canonical byte layout of one matrix: (packed [N, K/2], scale bits [N, G] as
    uint16, zeros [N, ceil(G/2)] or None), G = K / group."""
    if asymmetric:
        q, s, z = quantize_asym(w, group)
        return pack_nibbles(q), s.view(np.uint16), pack_nibbles(z)
    q, s = quantize_sym(w, group)
    return pack_nibbles(q), s.view(np.uint16), None


def unpack_canonical(packed, scale_bits, zeros_packed, k, asymmetric, group=GROUP):
    """Canonical bytes -> (q int64 [N, K], scales float16 [N, G], zeros int64 [N, G] or None)."""
    g = k // group
    q = unpack_nibbles(packed, k, signed=not asymmetric)
    s = np.asarray(scale_bits, dtype=np.uint16).view(np.float16)
    z = unpack_nibbles(zeros_packed, g, signed=False) if asymmetric else None
    return q, s, z


def packed_bytes(n, k, asymmetric, group=GROUP):
    """Bytes of the canonical format: N*K/2 nibble bytes + 2*N*G scale bytes
    (+ N*ceil(G/2) zero-point bytes), G = K / group."""
    g = k // group
    b = n * k // 2 + 2 * n * g
    if asymmetric:
        b += n * ((g + 1) // 2)
    return b
