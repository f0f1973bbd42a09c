"""Stage-by-stage checks of one MoE forward through moe_int4_ffn_debug (shared by the
stage-wise and full-size GPU tests); every reference is the oracle applied to the
GPU's own inputs of that stage."""
import numpy as np
import torch

import synth
from oracle import ffn, permute as operm
from tests.helpers import k_slice, y_positions


def _np(t):
    return synth.to_numpy(t)


def _rows_rel(y, ref):
    """per-row relative L2 (zero reference rows need zero rows)"""
    return ffn.max_rel_l2(y, ref)


# Per-row bar of a bf16-activation GEMM stage (W4A16 gate/up products, y) against the
# oracle's fp64 product on the same inputs.  The kernels widen a stored nibble d = q + 8
# to the bf16 value 128 + d and sum a * (136 + q) in fp32, removing 136 * sum(a) with the
# exact row sums afterwards: the fp32 rounding therefore scales with 136 * sum|a| rather
# than with |sum a * q|, about 30x a plain fp32 dot product's (measured up to 2.1e-5 per
# row with K = 128).  W4A8 stages accumulate in INT32, exactly, and keep 2e-5.
W4A16_STAGE_TOL = 1e-4


def gate_up_canonical(n2):
    """Device column c of a Q4_REPACK_GATE_UP block -> row of the stacked [gate; up]
    matrix: 16-column block 2b holds gate rows 16b.., block 2b + 1 up rows 16b.."""
    c = np.arange(n2)
    b, w = c // 16, c % 16
    return np.where(b % 2 == 0, 16 * (b // 2) + w, n2 // 2 + 16 * (b // 2) + w)


def expert_blocks(layer, e):
    E = layer.num_experts
    if e == E:
        return layer.shared_gate_up, layer.shared_down
    if layer.mixed:
        return (layer.gate_up[layer.gu_offs[e]:layer.gu_offs[e + 1]], layer.down[layer.dn_offs[e]:layer.dn_offs[e + 1]])
    return (layer.gate_up[e * layer.gu_bytes:(e + 1) * layer.gu_bytes],
            layer.down[e * layer.dn_bytes:(e + 1) * layer.dn_bytes])


def check_gate_up_core(lib, layer, e, mode, gate, up, a_rows, x32_rows, qx_rows):
    """gate and up of expert e on the given rows through the library's GEMM core on the
    layer's own gate/up block, against the oracle."""
    I = layer.inter
    gu_dev, _ = expert_blocks(layer, e)
    canon = gate_up_canonical(2 * I)
    if mode == 1:
        acc = _np(lib.int4_w4a8_group_acc(a_rows, gu_dev, 2 * I, layer.asymmetric))
        torch.cuda.synchronize()
        got = np.empty_like(acc)
        got[:, canon] = acc
        ref = np.concatenate([ffn.group_acc(qx_rows, ffn.widen_int8(gate)),
                              ffn.group_acc(qx_rows, ffn.widen_int8(up))], axis=1)
        assert np.array_equal(got, ref), f"gate/up group sums, expert {e}"
    else:
        y = _np(lib.int4_linear_forward(a_rows, gu_dev, 2 * I, layer.asymmetric)).astype(np.float64)
        torch.cuda.synchronize()
        got = np.empty_like(y)
        got[:, canon] = y
        ref = np.concatenate([ffn.linear_w4a16(x32_rows, gate), ffn.linear_w4a16(x32_rows, up)], axis=1)
        assert _rows_rel(got, ref) <= W4A16_STAGE_TOL, f"gate/up products, expert {e}"


def check_stagewise(lib, layer, oe, x, ids, w, mode, shared, expect_ksplit=None, experts=None, gate_up_rows=64):
    """Stage-by-stage checks of one forward; ``experts``: the experts whose positions are
    checked (all by default); ``gate_up_rows``: rows per expert given to the gate/up
    core checks."""
    t, k = ids.shape
    E = layer.num_experts
    plan = lib.moe_int4_ffn_plan(layer, t, mode)
    out, v = lib.moe_int4_ffn_debug(layer, x.cuda(), torch.as_tensor(ids, dtype=torch.int32).cuda(),
                                    torch.as_tensor(w, dtype=torch.float32).cuda(), mode=mode)
    torch.cuda.synchronize()
    S = v["slots_per_token"]
    assert S == k + (1 if shared else 0)
    assert v["y_slices"] == plan["down_ksplit"]
    if expect_ksplit is not None:
        assert v["y_slices"] == expect_ksplit, (v["y_slices"], expect_ksplit)
    # permutation over slots t * S + j (j == k: the shared expert)
    slot_ids = np.concatenate([ids, np.full((t, 1), E, np.int64)], axis=1) if shared else ids
    counts, offsets, perm, inv = operm.permute(slot_ids, E + (1 if shared else 0))
    assert np.array_equal(_np(v["counts"]), counts)
    assert np.array_equal(_np(v["offsets"]), offsets)
    assert np.array_equal(_np(v["perm"]), perm)
    assert np.array_equal(_np(v["inv"]), inv)
    x32 = _np(x).astype(np.float32)
    h = _np(v["h"]).astype(np.float64)
    ys = _np(v["y"]).astype(np.float64)          # [slices][P][H]
    y = y_positions(v)
    nsl, gsl, G = v["y_slices"], v["y_slice_groups"], layer.inter // 128
    if mode == 1:
        qx, sx = ffn.act_quant_int8(x32)
        assert np.array_equal(_np(v["q_x"]), qx)
        assert np.array_equal(_np(v["s_x"]).view(np.uint32), sx.view(np.uint32))
        qh_gpu, sh_gpu = _np(v["q_h"]), _np(v["s_h"])
        qh_ref, sh_ref = ffn.act_quant_int8(_np(v["h"]))
        assert np.array_equal(qh_gpu, qh_ref)
        assert np.array_equal(sh_gpu.view(np.uint32), sh_ref.view(np.uint32))
    for e in (range(E + (1 if shared else 0)) if experts is None else experts):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        toks = perm[lo:hi] // S
        gate, up, down = oe(e)
        _, dn_dev = expert_blocks(layer, e)
        sub = toks[:gate_up_rows]
        if mode == 1:
            check_gate_up_core(lib, layer, e, mode, gate, up, v["q_x"][torch.as_tensor(sub, dtype=torch.int64).cuda()].contiguous(),
                               None, qx[sub])
            g = ffn.linear_w4a8(qx[toks], sx[toks], gate)
            u = ffn.linear_w4a8(qx[toks], sx[toks], up)
            assert _rows_rel(h[lo:hi], ffn.silu(g) * u) <= 2e-5, f"h, expert {e}"
            # down-projection INT32 accumulators on the GPU's own h codes
            acc = lib.int4_w4a8_group_acc(v["q_h"][lo:hi].contiguous(), dn_dev, layer.hidden, layer.asymmetric)
            torch.cuda.synchronize()
            assert np.array_equal(_np(acc), ffn.group_acc(qh_gpu[lo:hi], ffn.widen_int8(down))), f"acc, expert {e}"
            down_of = lambda qm: ffn.linear_w4a8(qh_gpu[lo:hi], sh_gpu[lo:hi], qm)
            hk = None
        else:
            check_gate_up_core(lib, layer, e, mode, gate, up, x[torch.as_tensor(sub, dtype=torch.int64)].contiguous().cuda(),
                               x32[sub], None)
            g = ffn.linear_w4a16(x32[toks], gate)
            u = ffn.linear_w4a16(x32[toks], up)
            assert _rows_rel(h[lo:hi], ffn.silu(g) * u) <= 5e-3, f"h, expert {e}"
            down_of = lambda qm: ffn.linear_w4a16(hk, qm)
            hk = h[lo:hi]
        y_tol = 2e-5 if mode == 1 else W4A16_STAGE_TOL
        if nsl > 1:
            for sidx in range(nsl):
                g0, g1 = sidx * gsl, min(G, (sidx + 1) * gsl)
                assert g0 < g1, "empty K slice"
                if mode == 1:
                    ref_s = ffn.linear_w4a8(qh_gpu[lo:hi, 128 * g0:128 * g1], sh_gpu[lo:hi], k_slice(down, g0, g1))
                else:
                    ref_s = ffn.linear_w4a16(h[lo:hi, 128 * g0:128 * g1], k_slice(down, g0, g1))
                assert _rows_rel(ys[sidx, lo:hi], ref_s) <= y_tol, f"y slice {sidx}, expert {e}"
        assert _rows_rel(y[lo:hi], down_of(down)) <= y_tol, f"y, expert {e}"
    # combine of the GPU's per-position outputs
    ref = np.zeros((t, layer.hidden))
    for tok in range(t):
        for j in range(k):
            ref[tok] += w[tok, j] * y[inv[tok * S + j]]
        if shared:
            ref[tok] += y[inv[tok * S + k]]
    assert _rows_rel(_np(out), ref) <= 4e-3
    return out, v


