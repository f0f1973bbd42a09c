"""GPU parity of the W8A8 route (INT8 g128 weights, per-token INT8 activations)
against the oracle: quantisation, device layout and INT32 group accumulators bit-exact;
the MoE forward within 2e-2 per token (the W4A8 bar); stage by stage through
moe_int4_ffn_debug."""
import numpy as np
import pytest
import torch

import synth
from oracle import ffn, layout, quant, router
from oracle import permute as operm
from tests.helpers import random_expert_maker, require_gpu, y_positions

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module")
def lib():
    require_gpu()
    import int4_group_quantized_g128_amd as lib
    return lib


def _np(t):
    return synth.to_numpy(t)


def _special_weights(n, k, seed):
    w = synth.normal(synth.stream_key(seed, 78), (n, k), 0.02)
    w[0, :128] = 0.0
    w[1, :128] *= 1e-9
    w[2, 128:256] *= 1e-3
    w[3, :128] *= 1e5
    w[4, :128] = torch.abs(w[4, :128])
    return w


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("n,k", [(37, 384), (64, 2048)])
def test_quantize8_bit_exact(lib, dtype, n, k):
    w = _special_weights(n, k, 2).to(dtype)
    q, s = lib.quantize_int8_g128(w.cuda())
    rq, rs = quant.quantize_sym8(_np(w))
    assert np.array_equal(_np(q), rq)
    assert np.array_equal(_np(s).view(np.uint16), rs.view(np.uint16))


@pytest.mark.parametrize("gate_up", [False, True])
def test_repack8_bit_exact(lib, gate_up):
    n, k = 96, 640
    w = _special_weights(n, k, 3)
    q, s = lib.quantize_int8_g128(w.cuda())
    dev = lib.q8_repack_device(q, s, n, k, gate_up=gate_up)
    rq, rs = quant.quantize_sym8(_np(w))
    assert np.array_equal(_np(dev), layout.to_device8(rq, rs.view(np.uint16), n, k, gate_up))


@pytest.mark.parametrize("rows", [1, 19, 70])
def test_group_acc8_bit_exact(lib, rows):
    n, k = 128, 512
    w = synth.normal(synth.stream_key(79, n), (n, k), 0.05)
    q, s = lib.quantize_int8_g128(w.cuda())
    dev = lib.q8_repack_device(q, s, n, k)
    qa = torch.as_tensor(np.random.default_rng(rows).integers(-128, 128, (rows, k)), dtype=torch.int8)
    qa[0, :] = -128
    acc = lib.int8_w8a8_group_acc(qa.cuda(), dev, n)
    torch.cuda.synchronize()
    rq, _ = quant.quantize_sym8(_np(w))
    assert np.array_equal(_np(acc), ffn.group_acc(_np(qa), rq))


class Q8Experts:
    def __init__(self, make):
        self.make, self.cache = make, {}

    def __call__(self, e):
        if e not in self.cache:
            mats = self.make(e)
            self.cache[e] = tuple((lambda qs: (qs[0].astype(np.int64), qs[1], None))(quant.quantize_sym8(_np(m)))
                                  for m in mats)
        return self.cache[e]


def _layer8(lib, make, E, H, I, k, shared):
    layer = lib.MoELayer(E, H, I, k, shared=shared, weight_bits=8)
    for e in range(E + (1 if shared else 0)):
        g, u, d = make(e, "cuda")
        layer.set_expert(e, g, u, d)
    torch.cuda.synchronize()
    return layer


@pytest.fixture(scope="module")
def moe8(lib):
    cfg = synth.CONFIGS["moe8"]
    make = lambda e, device="cpu": synth.expert_weights("moe8", e, device)
    return _layer8(lib, make, cfg["experts"], cfg["hidden"], cfg["inter"], cfg["top_k"], False), Q8Experts(make)


@pytest.mark.parametrize("t", [40, 2048])
def test_moe8_w8a8(lib, moe8, t):
    layer, oe = moe8
    x = synth.tokens("moe8_w4a8", t)
    wr, b = synth.router_weights("moe8_w4a8")
    _, ids, w = router.route(_np(x), _np(wr), None, 2)
    out = lib.moe_int4_ffn_forward(layer, x.cuda(), torch.as_tensor(ids, dtype=torch.int32).cuda(),
                                   torch.as_tensor(w, dtype=torch.float32).cuda(), mode=lib.Q4_W8A8)
    torch.cuda.synchronize()
    rows = np.arange(t) if t <= 64 else np.sort(np.random.default_rng(8).choice(t, 48, replace=False))
    ref = ffn.moe_w8a8(_np(x)[rows], oe, ids[rows], w[rows])
    assert ffn.max_rel_l2(_np(out)[rows], ref) <= TOL


def test_mode_must_match_weight_bits(lib, moe8):
    layer, _ = moe8
    x = synth.tokens("moe8", 3)
    ids = torch.zeros((3, 2), dtype=torch.int32)
    ids[:, 1] = 1
    w = torch.full((3, 2), 0.5)
    with pytest.raises(lib.Q4Error):
        lib.moe_int4_ffn_forward(layer, x.cuda(), ids.cuda(), w.cuda(), mode=lib.Q4_W4A8)


@pytest.fixture(scope="module")
def small8(lib):
    make = random_expert_maker(81, 256, 128)
    return _layer8(lib, make, 16, 256, 128, 4, True), Q8Experts(make)


@pytest.mark.parametrize("t", [5, 300])
def test_small_shared_w8a8_stagewise(lib, small8, t):
    """End to end within 2e-2, and stage by stage: permutation, x / h codes and scales
    bit-exact, h and y within 2e-5 of the oracle on the GPU's own stage inputs, the
    down-projection INT32 group sums bit-exact on the GPU's h codes."""
    layer, oe = small8
    E, k, H = 16, 4, 256
    x = synth.normal(synth.stream_key(82, t), (t, H), 1.0).to(torch.bfloat16)
    rng = np.random.default_rng(t)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(t)]).astype(np.int64)
    w = rng.dirichlet(np.ones(k), size=t)
    out, v = lib.moe_int4_ffn_debug(layer, x.cuda(), torch.as_tensor(ids, dtype=torch.int32).cuda(),
                                    torch.as_tensor(w, dtype=torch.float32).cuda(), mode=lib.Q4_W8A8)
    torch.cuda.synchronize()
    ref = ffn.moe_w8a8(_np(x), oe, ids, w, shared=oe(E))
    assert ffn.max_rel_l2(_np(out), ref) <= TOL
    S = k + 1
    slot_ids = np.concatenate([ids, np.full((t, 1), E)], axis=1)
    counts, offsets, perm, inv = operm.permute(slot_ids, E + 1)
    assert np.array_equal(_np(v["perm"]), perm)
    qx, sx = ffn.act_quant_int8(_np(x).astype(np.float32))
    assert np.array_equal(_np(v["q_x"]), qx) and np.array_equal(_np(v["s_x"]).view(np.uint32), sx.view(np.uint32))
    h = _np(v["h"]).astype(np.float64)
    qh_gpu, sh_gpu = _np(v["q_h"]), _np(v["s_h"])
    qh_ref, sh_ref = ffn.act_quant_int8(_np(v["h"]))
    assert np.array_equal(qh_gpu, qh_ref) and np.array_equal(sh_gpu.view(np.uint32), sh_ref.view(np.uint32))
    y = y_positions(v)
    for e in range(E + 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        toks = perm[lo:hi] // S
        gate, up, down = oe(e)
        hr = ffn.silu(ffn.linear_w8a8(qx[toks], sx[toks], gate)) * ffn.linear_w8a8(qx[toks], sx[toks], up)
        assert ffn.max_rel_l2(h[lo:hi], hr) <= 2e-5
        wdev = layer.down[e * layer.dn_bytes:(e + 1) * layer.dn_bytes] if e < E else layer.shared_down
        acc = lib.int8_w8a8_group_acc(v["q_h"][lo:hi].contiguous(), wdev, H)
        torch.cuda.synchronize()
        assert np.array_equal(_np(acc), ffn.group_acc(qh_gpu[lo:hi], down[0]))
        assert ffn.max_rel_l2(y[lo:hi], ffn.linear_w8a8(qh_gpu[lo:hi], sh_gpu[lo:hi], down)) <= 2e-5


@pytest.mark.parametrize("t,ksplit", [(1, 4), (2, 2)])
def test_moe8_w8a8_ksplit(lib, moe8, t, ksplit):
    """T = 1 and 2 on the 8-expert layer: the down projection splits K (the 8-bit
    few-items kernel); every slice against the oracle's sum over its groups, and the
    output end to end."""
    from tests.helpers import k_slice
    layer, oe = moe8
    assert lib.moe_int4_ffn_plan(layer, t, lib.Q4_W8A8)["down_ksplit"] == ksplit
    x = synth.tokens("moe8", t)
    wr, _ = synth.router_weights("moe8")
    _, ids, w = router.route(_np(x), _np(wr), None, 2)
    out, v = lib.moe_int4_ffn_debug(layer, x.cuda(), torch.as_tensor(ids, dtype=torch.int32).cuda(),
                                    torch.as_tensor(w, dtype=torch.float32).cuda(), mode=lib.Q4_W8A8)
    torch.cuda.synchronize()
    assert ffn.max_rel_l2(_np(out), ffn.moe_w8a8(_np(x), oe, ids, w)) <= TOL
    assert v["y_slices"] == ksplit
    _, offsets, perm, _ = operm.permute(ids, 8)
    qh, sh = _np(v["q_h"]), _np(v["s_h"])
    ys = _np(v["y"]).astype(np.float64)
    gsl = v["y_slice_groups"]
    for e in range(8):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        down = oe(e)[2]
        for s in range(ksplit):
            g0, g1 = s * gsl, min(1024 // 128, (s + 1) * gsl)
            ref = ffn.linear_w8a8(qh[lo:hi, 128 * g0:128 * g1], sh[lo:hi], k_slice(down, g0, g1))
            assert ffn.max_rel_l2(ys[s, lo:hi], ref) <= 2e-5, (e, s)
        assert ffn.max_rel_l2(y_positions(v)[lo:hi], ffn.linear_w8a8(qh[lo:hi], sh[lo:hi], down)) <= 2e-5
