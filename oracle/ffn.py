"""FFN / MoE forward in W4A16 and W4A8 (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

A quantised matrix is the tuple (q, s, z): integer codes q [N, K] (int64),
binary16 scales s [N, K/128] and zero points z [N, K/128] (None for the
symmetric format).  Its real value is w_hat = (q - z) * s (quant.dequantize).

W4A16 (page "MoE推理优化实战：4bit存储+INT8计算的W4A8路线解析", §2.1: 4-bit
storage, computation in 16-bit after dequantisation; this build fuses the
dequantisation): every product is the exact real-number product with the
dequantised weights, evaluated in float64.

SwiGLU FFN (page "高效大语言模型推理实践：INT4量化与MoE架构的融合探索", 核心实现细节:
LLaMA 3.2 with a SwiGLU FFN): out = down(silu(gate x) * up x), silu(v) = v / (1 + e^-v).

MoE combine (page "大模型之Dense、MoE与量化", MoE section: expert outputs are
combined in proportion to the router scores; a shared expert is used by every
token): out[t] = sum_j w[t, j] * FFN_{ids[t, j]}(x[t]) (+ FFN_shared(x[t]) with
weight 1).

W4A8 (same W4A8 page, §2.3 three-step pipeline and §3.1 per-token activation
quantisation):

* activations are quantised per row: s = amax / 127 (float32 division),
  q = clamp(rint(x / s), -128, 127) (float32 division, half-to-even), a zero row
  gets s = 0 and q = 0;
* the 4-bit weight is widened to an 8-bit integer without scaling:
  w8 = q (symmetric) or q - z (asymmetric);
* INT32 accumulation per group: acc[t, n, g] = sum_{k in g} qx[t, k] * w8[n, k];
* rescale: y[t, n] = s_x[t] * sum_g s_w[n, g] * acc[t, n, g] (the pages'
  single scale_w * scale_a rescale, applied per group because the weight
  scales are per group);
* x is quantised once per token before gate/up, h once per (token, choice)
  row before down; the router stays in floating point.

Pinned by (tests/test_oracle_ffn.py): brute-force dense evaluation of every
expert on tiny inputs with an explicit per-token gather; the slice identity
(k = E, unit weights, sliced dense weights -> the dense FFN); E = 1 reduces to
the dense FFN; x = 0 -> 0; INT32 accumulators against element-by-element
integer sums and their |acc| bound; every non-zero row has a +-127 code; the
W4A8 special case (integer x with amax 127 -> s = 1 -> W4A8 gate/up equal
W4A16 gate/up).
"""
import numpy as np

from .quant import GROUP, dequantize, group_of


def silu(v):
    v = np.asarray(v, dtype=np.float64)
    return v / (1.0 + np.exp(-v))


# ---------------------------------------------------------------- W4A16
def linear_w4a16(x, qm):
    """y = x w_hat^T in float64."""
    q, s, z = qm
    return np.asarray(x, dtype=np.float64) @ dequantize(q, s, z).T


def swiglu_w4a16(x, gate, up, down):
    g = linear_w4a16(x, gate)
    u = linear_w4a16(x, up)
    return linear_w4a16(silu(g) * u, down)


def _routed_sum(ids, weights, hidden, expert_out, pmap=map):
    """out[t] = sum over the routed (t, j) of w[t, j] * y_{ids[t, j]}(x[t]): experts in
    ascending index, each expert's rows in token order.  ``expert_out(e, rows)`` gives
    the expert's outputs for those token rows; ``pmap`` may evaluate the (independent)
    experts concurrently -- the sums are still formed in the order above."""
    ids = np.asarray(ids)
    w = np.asarray(weights, dtype=np.float64)
    out = np.zeros((ids.shape[0], hidden), dtype=np.float64)
    experts = [int(e) for e in np.unique(ids)]
    where = [np.nonzero(ids == e) for e in experts]
    ys = list(pmap(lambda a: expert_out(a[0], a[1][0]), zip(experts, where)))
    for (rows, cols), y in zip(where, ys):
        for i, (r, c) in enumerate(zip(rows, cols)):
            out[r] += w[r, c] * y[i]
    return out


def moe_w4a16(x, expert, ids, weights, shared=None, pmap=map):
    """``expert(e)`` returns (gate, up, down) quantised matrices of expert e;
    ``shared`` is such a triple or None."""
    x64 = np.asarray(x, dtype=np.float64)
    out = _routed_sum(ids, weights, x64.shape[1], lambda e, rows: swiglu_w4a16(x64[rows], *expert(e)), pmap)
    if shared is not None:
        out += swiglu_w4a16(x64, *shared)
    return out


# ---------------------------------------------------------------- W4A8
def act_quant_int8(a):
    """Per-row symmetric INT8 quantisation in float32 (W4A8 page, §3.1)."""
    a32 = np.asarray(a, dtype=np.float32)
    amax = np.max(np.abs(a32), axis=1)
    s = amax / np.float32(127.0)                              # fp32 divide
    q = np.zeros(a32.shape, dtype=np.float32)
    nz = s > 0
    q[nz] = np.clip(np.rint(a32[nz] / s[nz][:, None]), -128, 127)
    return q.astype(np.int8), s.astype(np.float32)


def widen_int8(qm):
    """4-bit code -> 8-bit integer with the zero point removed, no scaling."""
    q, s, z = qm
    q = np.asarray(q, dtype=np.int64)
    if z is not None:
        q = q - np.repeat(np.asarray(z, dtype=np.int64), group_of(q.shape[1], s), axis=1)
    assert np.all(np.abs(q) <= 15)
    return q


def group_acc(qx, w8, group=GROUP):
    """acc[t, n, g] = sum_{k in group g} qx[t, k] * w8[n, k], exact (groups of
    ``group`` elements along K).

    The per-group products are evaluated by a float64 matrix product: every
    operand is an integer with |qx| <= 128 and |w8| <= 127 (<= 15 for 4-bit
    codes), so every partial sum is an integer below 128 * 128 * 127 < 2^53 and
    float64 represents it exactly.
    """
    qx = np.asarray(qx, dtype=np.int64)
    w8 = np.asarray(w8, dtype=np.int64)
    assert np.all(np.abs(qx) <= 128) and np.all(np.abs(w8) <= 127)
    t, k = qx.shape
    n = w8.shape[0]
    g = k // group
    qf = qx.astype(np.float64)
    wf = w8.astype(np.float64)
    acc = np.empty((t, n, g), dtype=np.int64)
    for gi in range(g):
        sl = slice(gi * group, (gi + 1) * group)
        acc[:, :, gi] = (qf[:, sl] @ wf[:, sl].T).astype(np.int64)
    return acc


def linear_w4a8(qx, sx, qm):
    """y[t, n] = s_x[t] * sum_g s_w[n, g] * acc[t, n, g] in float64."""
    q, s, _ = qm
    acc = group_acc(qx, widen_int8(qm), group_of(np.asarray(q).shape[1], s)).astype(np.float64)
    sw = np.asarray(s, dtype=np.float16).astype(np.float64)
    y = np.einsum("tng,ng->tn", acc, sw)
    return np.asarray(sx, dtype=np.float64)[:, None] * y


def swiglu_w4a8(x, gate, up, down, return_parts=False):
    qx, sx = act_quant_int8(x)
    g = linear_w4a8(qx, sx, gate)
    u = linear_w4a8(qx, sx, up)
    h = silu(g) * u
    qh, sh = act_quant_int8(h.astype(np.float32))
    y = linear_w4a8(qh, sh, down)
    if return_parts:
        return y, dict(qx=qx, sx=sx, g=g, u=u, h=h, qh=qh, sh=sh)
    return y


def moe_w4a8(x, expert, ids, weights, shared=None, pmap=map):
    x32 = np.asarray(x, dtype=np.float32)
    out = _routed_sum(ids, weights, x32.shape[1], lambda e, rows: swiglu_w4a8(x32[rows], *expert(e)), pmap)
    if shared is not None:
        out += swiglu_w4a8(x32, *shared)
    return out


# ---------------------------------------------------------------- W8A8
# The same pipeline with 8-bit weight codes (oracle/quant.quantize_sym8): no widening,
# INT32 group sums of int8(x) * q, rescale by s_x * s_w per group.
def linear_w8a8(qx, sx, qm):
    """y[t, n] = s_x[t] * sum_g s_w[n, g] * acc[t, n, g] in float64, 8-bit codes."""
    q, s, _ = qm
    acc = group_acc(qx, q).astype(np.float64)
    sw = np.asarray(s, dtype=np.float16).astype(np.float64)
    y = np.einsum("tng,ng->tn", acc, sw)
    return np.asarray(sx, dtype=np.float64)[:, None] * y


def swiglu_w8a8(x, gate, up, down):
    qx, sx = act_quant_int8(x)
    h = silu(linear_w8a8(qx, sx, gate)) * linear_w8a8(qx, sx, up)
    qh, sh = act_quant_int8(h.astype(np.float32))
    return linear_w8a8(qh, sh, down)


def moe_w8a8(x, expert, ids, weights, shared=None, pmap=map):
    x32 = np.asarray(x, dtype=np.float32)
    out = _routed_sum(ids, weights, x32.shape[1], lambda e, rows: swiglu_w8a8(x32[rows], *expert(e)), pmap)
    if shared is not None:
        out += swiglu_w8a8(x32, *shared)
    return out


# ---------------------------------------------------------------- mixed widths
# Per-expert weight precision (page "MoE推理优化实战：4bit存储+INT8计算的W4A8路线解析",
# §5.3 and §6.1: frequently hit / sensitive experts keep more bits; page "大模型之Dense、
# MoE与量化", APEX: precision by expert importance).  Every expert runs the INT8-activation
# pipeline above; an expert's own width picks the 4-bit (widened) or the 8-bit codes.
def swiglu_int8_acts(x, gate, up, down, bits):
    """SwiGLU FFN of one expert with INT8 activations and `bits`-wide weight codes (2 and 4
    bits: the codes are the 8-bit integers of the W4A8 pipeline as they are, no zero
    point; 8 bits: the W8A8 pipeline)."""
    return swiglu_w8a8(x, gate, up, down) if bits == 8 else swiglu_w4a8(x, gate, up, down)


def moe_mixed(x, expert, bits, ids, weights, shared=None, shared_bits=8, pmap=map):
    """out[t] = sum_j w[t, j] FFN_{ids[t, j]}(x[t]) (+ shared), expert e evaluated with
    bits[e]-wide weights; ``expert(e)`` returns its (gate, up, down) quantised matrices."""
    x32 = np.asarray(x, dtype=np.float32)
    out = _routed_sum(ids, weights, x32.shape[1],
                      lambda e, rows: swiglu_int8_acts(x32[rows], *expert(e), bits[e]), pmap)
    if shared is not None:
        out += swiglu_int8_acts(x32, *shared, shared_bits)
    return out


def bits_by_hotness(counts, frac8, shared=False):
    """Widths from hit counts: the ceil(frac8 * E) most-hit experts 8 bits (ties: lower
    index first), the others 4; a shared expert (hit by every token) 8."""
    counts = np.asarray(counts, dtype=np.int64)
    e = counts.shape[0]
    n8 = min(e, int(np.ceil(frac8 * e - 1e-9)))
    order = np.lexsort((np.arange(e), -counts))   # by count descending, then index
    bits = np.full(e, 4, dtype=np.int64)
    bits[order[:n8]] = 8
    return list(bits) + ([8] if shared else [])


def bits_apex(counts, frac8=0.0, cold_share=0.25, shared=False):
    """Widths 2 / 4 / 8 from hit counts (page "大模型之Dense、MoE与量化", APEX section:
    commonly used experts 4 bits, rarely used experts 2 bits; page "MoE推理优化实战：
    4bit存储+INT8计算的W4A8路线解析", §5.3: the most-hit experts keep more precision):
    experts hit less than cold_share times the even share (total / E) get 2 bits, the
    ceil(frac8 * E) most-hit experts (ties: lower index first) 8 bits -- over the cold
    rule --, the others 4; a shared expert (hit by every token) 8 bits if frac8 > 0,
    else 4."""
    counts = np.asarray(counts, dtype=np.int64)
    e = counts.shape[0]
    bits = np.full(e, 4, dtype=np.int64)
    bits[counts * e < cold_share * counts.sum()] = 2
    n8 = min(e, int(np.ceil(frac8 * e - 1e-9)))
    order = np.lexsort((np.arange(e), -counts))
    bits[order[:n8]] = 8
    return list(bits) + ([8 if frac8 > 0 else 4] if shared else [])


def groups_by_hotness(counts, hot_frac=0.05, cold_share=0.1, shared=False):
    """Group sizes from hit counts (page "MoE推理优化实战：4bit存储+INT8计算的W4A8路线解析",
    §5.3: the most-hit experts, its top 5 %, get groups of 32; ordinary experts 64;
    experts almost no token reaches 128 or even 256): the ceil(hot_frac * E) most-hit
    experts (ties: lower index first) 32; experts hit less than cold_share times the
    even share (total hits / E) 256; the others 64; a shared expert (hit by every
    token) 32."""
    counts = np.asarray(counts, dtype=np.int64)
    e = counts.shape[0]
    n_hot = min(e, int(np.ceil(hot_frac * e - 1e-9)))
    order = np.lexsort((np.arange(e), -counts))
    groups = np.full(e, 64, dtype=np.int64)
    groups[counts * e < cold_share * counts.sum()] = 256
    groups[order[:n_hot]] = 32
    return list(groups) + ([32] if shared else [])


# ---------------------------------------------------------------- comparison
def max_rel_l2(y, ref):
    """max over rows of ||y - ref||_2 / ||ref||_2; a zero reference row needs a zero row."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    worst = 0.0
    for a, b in zip(y, ref):
        nb = np.linalg.norm(b)
        if nb == 0.0:
            if np.linalg.norm(a) != 0.0:
                return np.inf
            continue
        worst = max(worst, np.linalg.norm(a - b) / nb)
    return worst
