"""GPU parity of the 2-bit cold-expert format (page "大模型之Dense、MoE与量化", APEX
section: commonly used experts 4 bits, rarely used ones 2 bits) against the oracle:
quantisation, device layout and INT32 group sums bit-exact; layers mixing 2-, 4- and
8-bit experts (INT8 activations) end to end within 2e-2 per token and stage by stage
(permutation, x / h codes and scales bit-exact, h and y within 2e-5 of the oracle on
the GPU's own stage inputs, the down projection's INT32 group sums bit-exact on each
expert's own device block), at decode sizes and at prefill sizes, where the 2-bit
experts' 128-row tiles run on the streaming kernel in 64-row sub-tiles."""
import numpy as np
import pytest
import torch

import synth
from oracle import ffn, layout, quant, router
from oracle import permute as operm
from tests.helpers import random_expert_maker, require_gpu, y_positions

pytestmark = pytest.mark.gpu
TOL = 2e-2
QUANT = {2: quant.quantize_sym2, 4: quant.quantize_sym, 8: quant.quantize_sym8}


@pytest.fixture(scope="module")
def lib():
    require_gpu()
    import int4_group_quantized_g128_amd as lib
    return lib


def _np(t):
    return synth.to_numpy(t)


def _special_weights(n, k, seed):
    w = synth.normal(synth.stream_key(seed, 77), (n, k), 0.02)
    w[0, :128] = 0.0
    w[1, :128] *= 1e-9           # below half the smallest subnormal scale: codes 0
    w[2, 128:256] *= 1e-3        # a subnormal scale
    w[3, :128] *= 1e5
    w[4, :128] = torch.abs(w[4, :128])
    w[5, :4] = torch.tensor([0.5, 0.25, -0.25, -0.5])   # exact ties at w / s = +-1/2
    w[5, 4:128] = 0.0
    return w


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("n,k", [(37, 384), (64, 2048)])
def test_quantize2_bit_exact(lib, dtype, n, k):
    w = _special_weights(n, k, 3).to(dtype)
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    p, s = lib.quantize_int2_g128(w.cuda(), flags)
    rq, rs = quant.quantize_sym2(_np(w))
    assert np.array_equal(_np(p), quant.pack_crumbs(rq))
    assert np.array_equal(_np(s).view(np.uint16), rs.view(np.uint16))
    assert int(flags.item()) == 0


def test_quantize2_flags_non_finite(lib):
    w = _special_weights(16, 256, 4)
    w[3, 7] = float("inf")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    lib.quantize_int2_g128(w.cuda(), flags)
    assert int(flags.item()) & 1


@pytest.mark.parametrize("gate_up", [False, True])
def test_repack2_bit_exact(lib, gate_up):
    n, k = 96, 640
    w = _special_weights(n, k, 5)
    p, s = lib.quantize_int2_g128(w.cuda())
    dev = lib.q2_repack_device(p, s, n, k, gate_up=gate_up)
    rq, rs = quant.quantize_sym2(_np(w))
    ref = layout.to_device2(quant.pack_crumbs(rq), rs.view(np.uint16), n, k, gate_up)
    assert np.array_equal(_np(dev), ref)


@pytest.mark.parametrize("rows", [1, 19, 70])
def test_group_acc2_bit_exact(lib, rows):
    n, k = 128, 512
    w = synth.normal(synth.stream_key(79, n), (n, k), 0.05)
    p, s = lib.quantize_int2_g128(w.cuda())
    dev = lib.q2_repack_device(p, s, n, k)
    qa = torch.as_tensor(np.random.default_rng(rows).integers(-128, 128, (rows, k)), dtype=torch.int8)
    qa[0, :] = -128
    acc = lib.int2_w2a8_group_acc(qa.cuda(), dev, n)
    torch.cuda.synchronize()
    rq, _ = quant.quantize_sym2(_np(w))
    assert np.array_equal(_np(acc), ffn.group_acc(_np(qa), rq))


class WidthExperts:
    """Oracle-quantised experts, each at its own width (2, 4 or 8 bits)."""

    def __init__(self, make, bits):
        self.make, self.bits, self.cache = make, bits, {}

    def __call__(self, e):
        if e not in self.cache:
            self.cache[e] = tuple((lambda qs: (qs[0].astype(np.int64), qs[1], None))(QUANT[self.bits[e]](_np(m)))
                                  for m in self.make(e))
        return self.cache[e]


def _layer(lib, make, E, H, I, k, shared, bits):
    layer = lib.MoELayer(E, H, I, k, shared=shared, expert_bits=bits)
    for e in range(E + (1 if shared else 0)):
        layer.set_expert(e, *make(e, "cuda"))
    torch.cuda.synchronize()
    return layer


SMALL_BITS = [2, 4, 4, 8, 2, 4, 2, 8, 4, 2, 2, 4, 4, 2, 4, 8, 4]   # 16 experts + shared


@pytest.fixture(scope="module")
def small(lib):
    make = random_expert_maker(191, 256, 128)
    return _layer(lib, make, 16, 256, 128, 4, True, SMALL_BITS), WidthExperts(make, SMALL_BITS)


def test_layer_bytes_follow_the_widths(lib, small):
    layer, _ = small
    sz = {2: (lib.q2_device_bytes(256, 256), lib.q2_device_bytes(256, 128)),
          4: (lib.q4_device_bytes(256, 256), lib.q4_device_bytes(256, 128)),
          8: (lib.q8_device_bytes(256, 256), lib.q8_device_bytes(256, 128))}
    assert layer.gate_up.numel() == sum(sz[b][0] for b in SMALL_BITS[:16])
    assert layer.down.numel() == sum(sz[b][1] for b in SMALL_BITS[:16])
    assert sz[2][0] == layout.device_bytes2(256, 256)


def _stagewise(lib, layer, oe, bits, x, ids, w, E, k, H):
    t = x.shape[0]
    out, v = lib.moe_int4_ffn_debug(layer, x.cuda(), torch.as_tensor(ids, dtype=torch.int32).cuda(),
                                    torch.as_tensor(w, dtype=torch.float32).cuda(), mode=lib.Q4_W4A8)
    torch.cuda.synchronize()
    ref = ffn.moe_mixed(_np(x), oe, bits, ids, w, shared=oe(E), shared_bits=bits[E])
    assert ffn.max_rel_l2(_np(out), ref) <= TOL
    S = k + 1
    slot_ids = np.concatenate([ids, np.full((t, 1), E)], axis=1)
    counts, offsets, perm, inv = operm.permute(slot_ids, E + 1)
    assert np.array_equal(_np(v["perm"]), perm) and np.array_equal(_np(v["inv"]), inv)
    qx, sx = ffn.act_quant_int8(_np(x).astype(np.float32))
    assert np.array_equal(_np(v["q_x"]), qx) and np.array_equal(_np(v["s_x"]).view(np.uint32), sx.view(np.uint32))
    qh_gpu, sh_gpu = _np(v["q_h"]), _np(v["s_h"])
    qh_ref, sh_ref = ffn.act_quant_int8(_np(v["h"]))
    assert np.array_equal(qh_gpu, qh_ref) and np.array_equal(sh_gpu.view(np.uint32), sh_ref.view(np.uint32))
    h = _np(v["h"]).astype(np.float64)
    y = y_positions(v)
    seen2 = 0
    for e in range(E + 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        toks = perm[lo:hi] // S
        gate, up, down = oe(e)
        lin = ffn.linear_w8a8 if bits[e] == 8 else ffn.linear_w4a8
        hr = ffn.silu(lin(qx[toks], sx[toks], gate)) * lin(qx[toks], sx[toks], up)
        assert ffn.max_rel_l2(h[lo:hi], hr) <= 2e-5, f"expert {e} ({bits[e]}-bit) h"
        wdev = layer.down[layer.dn_offs[e]:layer.dn_offs[e + 1]] if e < E else layer.shared_down
        qh_rows = v["q_h"][lo:hi].contiguous()
        if bits[e] == 8:
            acc = lib.int8_w8a8_group_acc(qh_rows, wdev, H)
        elif bits[e] == 2:
            acc = lib.int2_w2a8_group_acc(qh_rows, wdev, H)
            seen2 += hi - lo
        else:
            acc = lib.int4_w4a8_group_acc(qh_rows, wdev, H, False)
        torch.cuda.synchronize()
        assert np.array_equal(_np(acc), ffn.group_acc(qh_gpu[lo:hi], ffn.widen_int8(down) if bits[e] != 8
                                                       else down[0])), f"expert {e} down group sums"
        assert ffn.max_rel_l2(y[lo:hi], lin(qh_gpu[lo:hi], sh_gpu[lo:hi], down)) <= 2e-5, f"expert {e} y"
    assert seen2 > 0


@pytest.mark.parametrize("t", [5, 300])
def test_small_int2_stagewise(lib, small, t):
    """T = 5: decode tiles; T = 300 (about 75 rows per expert): prefill tiles, the 2-bit
    experts on the streaming kernel in 64-row sub-tiles of their 128-row tiles."""
    layer, oe = small
    E, k, H = 16, 4, 256
    assert lib.moe_int4_ffn_plan(layer, t, lib.Q4_W4A8)["kernel"] == ("prefill" if t == 300 else "decode")
    x = synth.normal(synth.stream_key(193, t), (t, H), 1.0).to(torch.bfloat16)
    rng = np.random.default_rng(t + 11)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(t)]).astype(np.int64)
    w = rng.dirichlet(np.ones(k), size=t)
    _stagewise(lib, layer, oe, SMALL_BITS, x, ids, w, E, k, H)


def test_all_two_bit_prefill_sub_tiles(lib):
    """Every expert 2-bit at a prefill size: some experts get more than 128 rows (two
    128-row tiles, each in two 64-row sub-tiles, the last ones part-filled or empty)."""
    make = random_expert_maker(194, 256, 128)
    E, k, H, t = 8, 2, 256, 700
    bits = [2] * (E + 1)
    layer = _layer(lib, make, E, H, 128, k, True, bits)
    oe = WidthExperts(make, bits)
    x = synth.normal(synth.stream_key(195, t), (t, H), 1.0).to(torch.bfloat16)
    rng = np.random.default_rng(196)
    p = np.array([0.4, 0.25, 0.15, 0.1, 0.05, 0.03, 0.015, 0.005])
    ids = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(t)]).astype(np.int64)
    w = rng.dirichlet(np.ones(k), size=t)
    assert lib.moe_int4_ffn_plan(layer, t, lib.Q4_W4A8)["kernel"] == "prefill"
    _stagewise(lib, layer, oe, bits, x, ids, w, E, k, H)


@pytest.fixture(scope="module")
def moe8(lib):
    """The 8-expert W4A8 workload with the APEX rule on a seeded calibration batch routed
    by the oracle: experts below 95 % of the even share (the load is nearly even here:
    the three least-hit experts) 2 bits, the others 4."""
    cfg = synth.CONFIGS["moe8_w4a8"]
    xc = _np(synth.tokens("moe8_w4a8", 2048, salt=7))
    wr, _ = synth.router_weights("moe8_w4a8")
    _, ids_c, _ = router.route(xc, _np(wr), None, 2)
    counts = np.bincount(ids_c.ravel(), minlength=8)
    bits = [int(b) for b in ffn.bits_apex(counts, 0.0, 0.95)]
    assert bits == lib.expert_bits_apex(counts.tolist(), 0.0, 0.95)
    assert sum(b == 2 for b in bits) == 3
    make = lambda e, device="cpu": synth.expert_weights("moe8", e, device)
    return _layer(lib, make, 8, cfg["hidden"], cfg["inter"], 2, False, bits), WidthExperts(make, bits), bits


@pytest.mark.parametrize("t", [1, 40, 2048])
def test_moe8_apex(lib, moe8, t):
    layer, oe, bits = moe8
    x = synth.tokens("moe8_w4a8", t)
    wr, _ = synth.router_weights("moe8_w4a8")
    _, ids, w = router.route(_np(x), _np(wr), None, 2)
    out = lib.moe_int4_ffn_forward(layer, x.cuda(), torch.as_tensor(ids, dtype=torch.int32).cuda(),
                                   torch.as_tensor(w, dtype=torch.float32).cuda(), mode=lib.Q4_W4A8)
    torch.cuda.synchronize()
    rows = np.arange(t) if t <= 64 else np.sort(np.random.default_rng(9).choice(t, 48, replace=False))
    ref = ffn.moe_mixed(_np(x)[rows], oe, bits, ids[rows], w[rows])
    assert ffn.max_rel_l2(_np(out)[rows], ref) <= TOL
