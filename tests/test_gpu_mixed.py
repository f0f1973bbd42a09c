"""GPU parity of mixed-width layers (each expert's weights in INT4 or INT8 g128 codes,
INT8 activations everywhere) against the oracle (oracle/ffn.moe_mixed): end to end
within 2e-2 per token (the W4A8 bar), and stage by stage on the small layer: the
permutation, the x / h codes and scales bit-exact, h and y within 2e-5 of the oracle on
the GPU's own stage inputs, the down projection's INT32 group sums bit-exact on each
expert's own device block."""
import numpy as np
import pytest
import torch

import synth
from oracle import ffn, quant, router
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


class MixedExperts:
    """Oracle-quantised experts, each at its own width."""

    def __init__(self, make, bits):
        self.make, self.bits, self.cache = make, bits, {}

    def __call__(self, e):
        if e not in self.cache:
            out = []
            for m in self.make(e):
                w = _np(m)
                q, s = quant.quantize_sym8(w) if self.bits[e] == 8 else quant.quantize_sym(w)
                out.append((q.astype(np.int64), s, None))
            self.cache[e] = tuple(out)
        return self.cache[e]


def _layer(lib, make, E, H, I, k, shared, bits):
    layer = lib.MoELayer(E, H, I, k, shared=shared, expert_bits=bits)
    for e in range(E + (1 if shared else 0)):
        layer.set_expert(e, *make(e, "cuda"))
    torch.cuda.synchronize()
    return layer


SMALL_BITS = [8, 4, 4, 8, 4, 4, 4, 8, 4, 4, 8, 4, 4, 4, 4, 8, 8]   # 16 experts + shared


@pytest.fixture(scope="module")
def small(lib):
    make = random_expert_maker(91, 256, 128)
    return _layer(lib, make, 16, 256, 128, 4, True, SMALL_BITS), MixedExperts(make, SMALL_BITS)


def test_layer_bytes_follow_the_widths(lib, small):
    layer, _ = small
    gu4, gu8 = lib.q4_device_bytes(256, 256, False), lib.q8_device_bytes(256, 256)
    dn4, dn8 = lib.q4_device_bytes(256, 128, False), lib.q8_device_bytes(256, 128)
    n8 = sum(b == 8 for b in SMALL_BITS[:16])
    assert layer.gate_up.numel() == n8 * gu8 + (16 - n8) * gu4
    assert layer.down.numel() == n8 * dn8 + (16 - n8) * dn4
    assert layer.shared_gate_up.numel() == gu8 and layer.shared_down.numel() == dn8
    assert all(o % 256 == 0 for o in layer.gu_offs + layer.dn_offs)


def test_mixed_layer_refuses_other_modes(lib, small):
    layer, _ = small
    x = synth.normal(synth.stream_key(92), (3, 256), 1.0).to(torch.bfloat16)
    ids = torch.tensor([[0, 1, 2, 3]] * 3, dtype=torch.int32)
    w = torch.full((3, 4), 0.25)
    for mode in (lib.Q4_W4A16, lib.Q4_W8A8):
        with pytest.raises(lib.Q4Error):
            lib.moe_int4_ffn_forward(layer, x.cuda(), ids.cuda(), w.cuda(), mode=mode)


@pytest.mark.parametrize("t", [5, 300])
def test_small_mixed_stagewise(lib, small, t):
    """T = 5 runs the decode GEMMs, T = 300 (about 88 rows per expert) the prefill GEMMs."""
    layer, oe = small
    E, k, H = 16, 4, 256
    x = synth.normal(synth.stream_key(93, t), (t, H), 1.0).to(torch.bfloat16)
    rng = np.random.default_rng(t + 1)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(t)]).astype(np.int64)
    w = rng.dirichlet(np.ones(k), size=t)
    out, v = lib.moe_int4_ffn_debug(layer, x.cuda(), torch.as_tensor(ids, dtype=torch.int32).cuda(),
                                    torch.as_tensor(w, dtype=torch.float32).cuda(), mode=lib.Q4_W4A8)
    torch.cuda.synchronize()
    ref = ffn.moe_mixed(_np(x), oe, SMALL_BITS, ids, w, shared=oe(E), shared_bits=SMALL_BITS[E])
    assert ffn.max_rel_l2(_np(out), ref) <= TOL
    S = k + 1
    slot_ids = np.concatenate([ids, np.full((t, 1), E)], axis=1)
    _, offsets, perm, _ = operm.permute(slot_ids, E + 1)
    assert np.array_equal(_np(v["perm"]), perm)
    qx, sx = ffn.act_quant_int8(_np(x).astype(np.float32))
    assert np.array_equal(_np(v["q_x"]), qx) and np.array_equal(_np(v["s_x"]).view(np.uint32), sx.view(np.uint32))
    qh_gpu, sh_gpu = _np(v["q_h"]), _np(v["s_h"])
    qh_ref, sh_ref = ffn.act_quant_int8(_np(v["h"]))
    assert np.array_equal(qh_gpu, qh_ref) and np.array_equal(sh_gpu.view(np.uint32), sh_ref.view(np.uint32))
    h = _np(v["h"]).astype(np.float64)
    y = y_positions(v)
    for e in range(E + 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        toks = perm[lo:hi] // S
        gate, up, down = oe(e)
        lin = ffn.linear_w8a8 if SMALL_BITS[e] == 8 else ffn.linear_w4a8
        hr = ffn.silu(lin(qx[toks], sx[toks], gate)) * lin(qx[toks], sx[toks], up)
        assert ffn.max_rel_l2(h[lo:hi], hr) <= 2e-5, f"expert {e} ({SMALL_BITS[e]}-bit) h"
        wdev = layer.down[layer.dn_offs[e]:layer.dn_offs[e + 1]] if e < E else layer.shared_down
        if SMALL_BITS[e] == 8:
            acc = lib.int8_w8a8_group_acc(v["q_h"][lo:hi].contiguous(), wdev, H)
            w8 = down[0]
        else:
            acc = lib.int4_w4a8_group_acc(v["q_h"][lo:hi].contiguous(), wdev, H, False)
            w8 = ffn.widen_int8(down)
        torch.cuda.synchronize()
        assert np.array_equal(_np(acc), ffn.group_acc(qh_gpu[lo:hi], w8)), f"expert {e} down group sums"
        assert ffn.max_rel_l2(y[lo:hi], lin(qh_gpu[lo:hi], sh_gpu[lo:hi], down)) <= 2e-5, f"expert {e} y"


@pytest.fixture(scope="module")
def moe8(lib):
    cfg = synth.CONFIGS["moe8"]
    bits = [8, 4, 4, 4, 4, 8, 4, 4]
    make = lambda e, device="cpu": synth.expert_weights("moe8", e, device)
    layer = _layer(lib, make, cfg["experts"], cfg["hidden"], cfg["inter"], cfg["top_k"], False, bits)
    return layer, MixedExperts(make, bits), bits


@pytest.mark.parametrize("t", [40, 2048])
def test_moe8_mixed(lib, moe8, t):
    """The W4A8 prefill workload (1 % hot channels x10) with two of the eight experts in
    8 bits; at T = 2048 a seeded sample of tokens is checked."""
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


def test_all_four_bit_mixed_equals_uniform_w4a8(lib, small):
    """A mixed layer whose experts are all 4-bit gives the uniform INT4 layer's W4A8 result
    bit for bit (same kernels, the 8-bit launch skips every tile)."""
    make = random_expert_maker(94, 256, 128)
    E, H, I, k, t = 8, 256, 128, 2, 70
    mixed = _layer(lib, make, E, H, I, k, False, [4] * E)
    uni = lib.MoELayer(E, H, I, k)
    for e in range(E):
        uni.set_expert(e, *make(e, "cuda"))
    x = synth.normal(synth.stream_key(95, t), (t, H), 1.0).to(torch.bfloat16).cuda()
    rng = np.random.default_rng(96)
    ids = torch.as_tensor(np.stack([rng.permutation(E)[:k] for _ in range(t)]), dtype=torch.int32).cuda()
    w = torch.as_tensor(rng.dirichlet(np.ones(k), size=t), dtype=torch.float32).cuda()
    a = lib.moe_int4_ffn_forward(mixed, x, ids, w, mode=lib.Q4_W4A8)
    b = lib.moe_int4_ffn_forward(uni, x, ids, w, mode=lib.Q4_W4A8)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
