"""GPU parity of LoRA-mode experts (moe_lora_ffn_forward) against the fp64 oracle
(oracle/lora.py): per-token max relative L2 <= 5e-3 (bf16 output; h summed over the
token's choices in fp32 and rounded to bf16 once, as for the W4A16 path)."""
import numpy as np
import pytest
import torch

import synth
from oracle import ffn, lora, quant, router
from tests.helpers import require_gpu

pytestmark = pytest.mark.gpu
TOL = 5e-3


@pytest.fixture(scope="module")
def lib():
    require_gpu()
    import int4_group_quantized_g128_amd as lib
    return lib


def _np(t):
    return synth.to_numpy(t)


def _qm(w, asym):
    w = _np(w)
    if asym:
        q, s, z = quant.quantize_asym(w)
        return q.astype(np.int64), s, z.astype(np.int64)
    q, s = quant.quantize_sym(w)
    return q.astype(np.int64), s, None


def _build(lib, base, adapters, E, H, I, k, r, asym):
    layer = lib.LoRALayer(E, H, I, k, r, asymmetric=asym)
    layer.set_base(*(m.cuda() for m in base))
    for e in range(E):
        layer.set_adapters(e, {n: v.cuda() for n, v in adapters(e).items()})
    torch.cuda.synchronize()
    oracle_base = tuple(_qm(m, asym) for m in base)
    oracle_ad = lambda e: {n: _np(v).astype(np.float64) for n, v in adapters(e).items()}
    return layer, oracle_base, oracle_ad


def _route(t, E, k, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(t)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), size=t)
    return ids, w


def _run(lib, layer, x, ids, w):
    out = lib.moe_lora_ffn_forward(layer, x.cuda(), torch.as_tensor(ids, dtype=torch.int32).cuda(),
                                   torch.as_tensor(w, dtype=torch.float32).cuda())
    torch.cuda.synchronize()
    return out


SMALL = dict(E=4, H=256, I=384, k=2, r=8)


@pytest.fixture(scope="module", params=[False, True], ids=["sym", "asym"])
def small(lib, request):
    asym = request.param
    E, H, I, k, r = (SMALL[n] for n in ("E", "H", "I", "k", "r"))
    base = (synth.normal(synth.stream_key(61, 1), (I, H), 0.05), synth.normal(synth.stream_key(61, 2), (I, H), 0.05),
            synth.normal(synth.stream_key(61, 3), (H, I), 0.05))
    adapters = lambda e: synth.lora_adapters("lora8", e, rank=r, dims=(H, I))
    return _build(lib, base, adapters, E, H, I, k, r, asym)


@pytest.mark.parametrize("t", [1, 5, 70, 200])
def test_small_lora_layer(lib, small, t):
    layer, ob, oa = small
    x = synth.normal(synth.stream_key(62, t), (t, SMALL["H"]), 1.0).to(torch.bfloat16)
    ids, w = _route(t, SMALL["E"], SMALL["k"], t)
    out = _run(lib, layer, x, ids, w)
    ref = lora.moe_lora(_np(x), ob, oa, ids, w)
    assert ffn.max_rel_l2(_np(out), ref) <= TOL


def test_zero_adapters_equal_dense(lib, small):
    """Adapters zero: every expert is the dense INT4 FFN, so the output is the dense
    FFN's whatever the routing (weights sum to 1)."""
    layer, ob, _ = small
    E, H, I, k, r = (SMALL[n] for n in ("E", "H", "I", "k", "r"))
    zero = lib.LoRALayer(E, H, I, k, r, asymmetric=layer.asymmetric)
    zero.base_gate_up.copy_(layer.base_gate_up)
    zero.base_down.copy_(layer.base_down)
    t = 9
    x = synth.normal(synth.stream_key(63, t), (t, H), 1.0).to(torch.bfloat16)
    ids, w = _route(t, E, k, 3)
    out = _run(lib, zero, x, ids, w)
    assert ffn.max_rel_l2(_np(out), ffn.swiglu_w4a16(_np(x), *ob)) <= TOL


@pytest.mark.parametrize("r", [24, 40, 64])
def test_lora_ranks(lib, r):
    """Ranks above 16: the adapter kernels load the rows of two columns or one at a time
    and the down-adapter rows 16 at a time (rank 16 and below load everything at once)."""
    E, H, I, k = 4, 256, 384, 2
    base = (synth.normal(synth.stream_key(64, 1), (I, H), 0.05), synth.normal(synth.stream_key(64, 2), (I, H), 0.05),
            synth.normal(synth.stream_key(64, 3), (H, I), 0.05))
    adapters = lambda e: synth.lora_adapters("lora8", e, rank=r, dims=(H, I))
    layer, ob, oa = _build(lib, base, adapters, E, H, I, k, r, False)
    for t in (3, 70):
        x = synth.normal(synth.stream_key(65, t, r), (t, H), 1.0).to(torch.bfloat16)
        ids, w = _route(t, E, k, t + r)
        out = _run(lib, layer, x, ids, w)
        ref = lora.moe_lora(_np(x), ob, oa, ids, w)
        assert ffn.max_rel_l2(_np(out), ref) <= TOL, (r, t)


@pytest.mark.parametrize("r", [16, 32])
@pytest.mark.parametrize("t", [256, 300])
def test_lora_grouped_by_expert(lib, r, t):
    """From 256 tokens, ranks 16 and 32 run the adapter work grouped by expert (tiles of
    at most 64 routed slots of one expert); I = 384 leaves a ragged second block of 256
    columns and T = 300 ragged tiles."""
    E, H, I, k = 4, 256, 384, 2
    base = (synth.normal(synth.stream_key(66, 1), (I, H), 0.05), synth.normal(synth.stream_key(66, 2), (I, H), 0.05),
            synth.normal(synth.stream_key(66, 3), (H, I), 0.05))
    adapters = lambda e: synth.lora_adapters("lora8", e, rank=r, dims=(H, I))
    layer, ob, oa = _build(lib, base, adapters, E, H, I, k, r, r == 32)
    x = synth.normal(synth.stream_key(67, t, r), (t, H), 1.0).to(torch.bfloat16)
    ids, w = _route(t, E, k, t + 3 * r)
    out = _run(lib, layer, x, ids, w)
    ref = lora.moe_lora(_np(x), ob, oa, ids, w)
    assert ffn.max_rel_l2(_np(out), ref) <= TOL, (r, t)


@pytest.fixture(scope="module")
def lora8(lib):
    cfg = synth.CONFIGS["lora8"]
    base = synth.lora_base("lora8")
    adapters = lambda e: synth.lora_adapters("lora8", e)
    return _build(lib, base, adapters, cfg["experts"], cfg["hidden"], cfg["inter"], cfg["top_k"], cfg["rank"], False)


@pytest.mark.parametrize("t", [1, 64, 300])
def test_lora8(lib, lora8, t):
    """The 8-expert rank-16 layer on the 2048/8192 dense FFN, routed by its router; at
    T = 300 the oracle checks a seeded sample of 24 tokens."""
    layer, ob, oa = lora8
    cfg = synth.CONFIGS["lora8"]
    x = synth.tokens("lora8", t)
    wr, b = synth.router_weights("lora8")
    _, ids, w = router.route(_np(x), _np(wr), None, cfg["top_k"])
    out = _run(lib, layer, x, ids, w)
    rows = np.arange(t) if t <= 64 else np.sort(np.random.default_rng(7).choice(t, 24, replace=False))
    ref = lora.moe_lora(_np(x)[rows], ob, oa, ids[rows], w[rows])
    assert ffn.max_rel_l2(_np(out)[rows], ref) <= TOL


def test_lora_grouped_many_experts(lib):
    """Grouped adapter path with many experts and four choices per token (E = 64,
    top-4, rank 16, T = 320): most tiles of the permutation hold a few slots, some
    experts none."""
    E, H, I, k, r, t = 64, 256, 384, 4, 16, 320
    base = (synth.normal(synth.stream_key(68, 1), (I, H), 0.05), synth.normal(synth.stream_key(68, 2), (I, H), 0.05),
            synth.normal(synth.stream_key(68, 3), (H, I), 0.05))
    adapters = lambda e: synth.lora_adapters("lora8", e, rank=r, dims=(H, I))
    layer, ob, oa = _build(lib, base, adapters, E, H, I, k, r, False)
    x = synth.normal(synth.stream_key(69, t), (t, H), 1.0).to(torch.bfloat16)
    rng = np.random.default_rng(5)
    ids = np.stack([rng.choice(E // 2, k, replace=False) for _ in range(t)]).astype(np.int32)   # experts 32.. unused
    w = rng.dirichlet(np.ones(k), size=t)
    out = _run(lib, layer, x, ids, w)
    ref = lora.moe_lora(_np(x), ob, oa, ids, w)
    assert ffn.max_rel_l2(_np(out), ref) <= TOL
