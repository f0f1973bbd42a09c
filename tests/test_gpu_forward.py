"""GPU parity of the MoE / FFN forward (W4A16, W4A8) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import synth
from oracle import ffn, router
from tests.helpers import OracleExperts, build_gpu_layer, random_expert_maker, require_gpu

pytestmark = pytest.mark.gpu

TOL_W4A16 = 5e-3
TOL_W4A8 = 2e-2


@pytest.fixture(scope="module")
def lib():
    require_gpu()
    import int4_group_quantized_g128_amd as lib
    return lib


def _np(t):
    return synth.to_numpy(t)


def _forward(lib, layer, x, ids, w, mode):
    out = lib.moe_int4_ffn_forward(layer, x.cuda(), torch.as_tensor(ids, dtype=torch.int32).cuda(),
                                   torch.as_tensor(w, dtype=torch.float32).cuda(), mode=mode)
    torch.cuda.synchronize()
    return out


def _oracle_route(x, name):
    cfg = synth.CONFIGS[name]
    w, b = synth.router_weights(name)
    _, ids, wts = router.route(_np(x), _np(w), _np(b) if b is not None else None, cfg["top_k"])
    return ids, wts


# ------------------------------------------------------------------ small layer with a shared expert
SMALL = dict(e=16, h=256, i=128, k=4)


@pytest.fixture(scope="module", params=[False, True], ids=["sym", "asym"])
def small(lib, request):
    asym = request.param
    make = random_expert_maker(11 + asym, SMALL["h"], SMALL["i"])
    layer = build_gpu_layer(lib, make, SMALL["e"], SMALL["h"], SMALL["i"], SMALL["k"], asym=asym, shared=True)
    return layer, OracleExperts(make, asym)


@pytest.mark.parametrize("mode", [0, 1], ids=["w4a16", "w4a8"])
@pytest.mark.parametrize("t", [1, 5, 33, 100, 300])
def test_small_shared_layer(lib, small, mode, t):
    layer, oe = small
    x = synth.normal(synth.stream_key(12, t), (t, SMALL["h"]), 1.0).to(torch.bfloat16)
    rng = np.random.default_rng(t)
    ids = np.stack([rng.permutation(SMALL["e"])[: SMALL["k"]] for _ in range(t)]).astype(np.int32)
    L = rng.normal(size=(t, SMALL["e"]))
    w = np.take_along_axis(np.exp(L), ids.astype(np.int64), axis=1)
    w /= w.sum(axis=1, keepdims=True)
    out = _forward(lib, layer, x, ids, w, mode)
    fn = ffn.moe_w4a16 if mode == 0 else ffn.moe_w4a8
    ref = fn(_np(x), oe, ids, w, shared=oe(SMALL["e"]))
    assert ffn.max_rel_l2(_np(out), ref) <= (TOL_W4A16 if mode == 0 else TOL_W4A8)


@pytest.mark.parametrize("mode", [0, 1], ids=["w4a16", "w4a8"])
@pytest.mark.parametrize("t", [3, 40])
def test_hidden_not_a_multiple_of_256(lib, mode, t):
    """Hidden 384: the down projection's 16-row decode tiles cannot take the 256-column
    bf16 workgroups (384 = 1.5 x 256) and fall back to the narrow configuration; int8's
    128-column workgroups divide it.  6 experts x inter 128, top-2, shared expert."""
    E, H, I, k = 6, 384, 128, 2
    make = random_expert_maker(17, H, I)
    layer = build_gpu_layer(lib, make, E, H, I, k, shared=True)
    oe = OracleExperts(make, False)
    x = synth.normal(synth.stream_key(18, t), (t, H), 1.0).to(torch.bfloat16)
    rng = np.random.default_rng(19 + t)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(t)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), size=t)
    out = _forward(lib, layer, x, ids, w, mode)
    fn = ffn.moe_w4a16 if mode == 0 else ffn.moe_w4a8
    ref = fn(_np(x), oe, ids, w, shared=oe(E))
    assert ffn.max_rel_l2(_np(out), ref) <= (TOL_W4A16 if mode == 0 else TOL_W4A8)


def test_zero_tokens_is_noop(lib, small):
    layer, _ = small
    x = torch.zeros((0, SMALL["h"]), dtype=torch.bfloat16)
    out = _forward(lib, layer, x, np.zeros((0, SMALL["k"])), np.zeros((0, SMALL["k"])), 0)
    assert out.shape == (0, SMALL["h"])


def test_zero_input_gives_zero_output(lib, small):
    layer, _ = small
    x = torch.zeros((7, SMALL["h"]), dtype=torch.bfloat16)
    ids = np.tile(np.arange(SMALL["k"], dtype=np.int32), (7, 1))
    w = np.full((7, SMALL["k"]), 1.0 / SMALL["k"])
    for mode in (0, 1):
        assert torch.count_nonzero(_forward(lib, layer, x, ids, w, mode)) == 0


def test_hot_expert_and_deterministic(lib, small):
    layer, oe = small
    t = 150
    x = synth.normal(synth.stream_key(13, t), (t, SMALL["h"]), 1.0).to(torch.bfloat16)
    ids = np.tile(np.array([3, 0, 9, 15], dtype=np.int32), (t, 1))   # every token on the same experts
    w = np.tile(np.array([0.4, 0.3, 0.2, 0.1]), (t, 1))
    a = _forward(lib, layer, x, ids, w, 0)
    b = _forward(lib, layer, x, ids, w, 0)
    assert torch.equal(a, b)
    ref = ffn.moe_w4a16(_np(x), oe, ids, w, shared=oe(SMALL["e"]))
    assert ffn.max_rel_l2(_np(a), ref) <= TOL_W4A16


# ------------------------------------------------------------------ dense SwiGLU FFN (E = 1)
@pytest.fixture(scope="module")
def dense(lib):
    cfg = synth.CONFIGS["dense"]
    g, u, d = synth.dense_ffn_weights("dense")
    layer = lib.MoELayer(1, cfg["hidden"], cfg["inter"], 1, asymmetric=True)
    layer.set_expert(0, g.cuda(), u.cuda(), d.cuda())
    torch.cuda.synchronize()
    oe = OracleExperts(lambda e: (g, u, d), True)
    return layer, oe


@pytest.mark.parametrize("t", [1, 4, 16])
def test_dense_ffn_asym_w4a16(lib, dense, t):
    layer, oe = dense
    x = synth.tokens("dense", t)
    ids = np.zeros((t, 1), np.int32)
    w = np.ones((t, 1))
    out = _forward(lib, layer, x, ids, w, 0)
    ref = ffn.swiglu_w4a16(_np(x), *oe(0))
    assert ffn.max_rel_l2(_np(out), ref) <= TOL_W4A16


def test_dense_ffn_asym_w4a8(lib, dense):
    layer, oe = dense
    x = synth.tokens("dense", 16)
    out = _forward(lib, layer, x, np.zeros((16, 1), np.int32), np.ones((16, 1)), 1)
    ref = ffn.swiglu_w4a8(_np(x), *oe(0))
    assert ffn.max_rel_l2(_np(out), ref) <= TOL_W4A8


@pytest.mark.parametrize("mode", [0, 1], ids=["w4a16", "w4a8"])
@pytest.mark.parametrize("t", [1, 4, 16, 17, 40, 63])
def test_dense_one_expert_path(lib, dense, t, mode):
    """The one-expert decode path: no permutation launch, rows in token order; from 17
    tokens (no K slices) the down projection applies the weight and rounds to bf16 in its
    epilogue.  Weights other than 1 (the combine's multiply is exercised); the result
    equals the debug call's (which runs the permutation and the separate combine) bit for
    bit, also on repeated calls with a workspace of nonzero bytes, and the oracle within
    the mode's bar."""
    layer, oe = dense
    plan = lib.moe_int4_ffn_plan(layer, t, mode)
    assert plan["kernel"] == "decode" and plan["rows_in_token_order"]
    assert plan["combine_in_down"] == (t > 16) and (plan["down_ksplit"] > 1) == (t <= 16)
    x = synth.tokens("dense", t)
    ids = np.zeros((t, 1), np.int32)
    w = np.random.default_rng(t).uniform(0.25, 1.75, (t, 1))
    out = _forward(lib, layer, x, ids, w, mode)
    # a workspace full of nonzero bytes, twice: no step depends on its prior contents
    ws = torch.full((layer.workspace_bytes(t, mode),), 0x5A, dtype=torch.uint8, device="cuda")
    args = (x.cuda(), torch.as_tensor(ids).cuda(), torch.as_tensor(w, dtype=torch.float32).cuda())
    again = [lib.moe_int4_ffn_forward(layer, *args, mode=mode, workspace=ws) for _ in range(2)]
    dbg, _ = lib.moe_int4_ffn_debug(layer, *args, mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), dbg.cpu())
    assert all(torch.equal(a.cpu(), out.cpu()) for a in again)
    ref = (ffn.moe_w4a16 if mode == 0 else ffn.moe_w4a8)(_np(x), oe, ids, w)
    assert ffn.max_rel_l2(_np(out), ref) <= (TOL_W4A16 if mode == 0 else TOL_W4A8)


# ------------------------------------------------------------------ 8 experts, top-2 (slice mode)
@pytest.fixture(scope="module")
def moe8(lib):
    cfg = synth.CONFIGS["moe8"]
    make = lambda e, device="cpu": synth.expert_weights("moe8", e, device)
    layer = build_gpu_layer(lib, make, cfg["experts"], cfg["hidden"], cfg["inter"], cfg["top_k"])
    return layer, OracleExperts(make, False)


@pytest.mark.parametrize("t", [1, 2, 16, 64, 256])
def test_moe8_w4a16(lib, moe8, t):
    layer, oe = moe8
    x = synth.tokens("moe8", t)
    ids, w = _oracle_route(x, "moe8")
    out = _forward(lib, layer, x, ids, w, 0)
    ref = ffn.moe_w4a16(_np(x), oe, ids, w)
    assert ffn.max_rel_l2(_np(out), ref) <= TOL_W4A16


def test_moe8_slice_identity(lib, moe8):
    """k = E with unit weights reproduces the dense FFN the experts were sliced from."""
    layer, _ = moe8
    cfg = synth.CONFIGS["moe8"]
    t = 8
    x = synth.tokens("moe8", t, salt=5)
    ids = np.tile(np.arange(8, dtype=np.int32), (t, 1))
    # a layer with top_k = 8 over the same weights
    full = type(layer).__new__(type(layer))
    full.__dict__.update(layer.__dict__)
    full.top_k = 8
    full.desc = type(layer.desc)(8, cfg["hidden"], cfg["inter"], 8, 0, 0, layer.gate_up.data_ptr(),
                                 layer.down.data_ptr(), None, None)
    out = _forward(lib, full, x, ids, np.ones((t, 8)), 0)
    g, u, d = synth.dense_ffn_weights("moe8")
    from tests.helpers import oracle_qmat
    ref = ffn.swiglu_w4a16(_np(x), oracle_qmat(g, False), oracle_qmat(u, False), oracle_qmat(d, False))
    assert ffn.max_rel_l2(_np(out), ref) <= TOL_W4A16


@pytest.mark.parametrize("t", [40, 2048])
def test_moe8_w4a8(lib, moe8, t):
    """The W4A8 prefill workload (1 % hot channels x10); at T = 2048 the oracle checks a
    seeded sample of tokens (tokens are independent given the routing)."""
    layer, oe = moe8
    x = synth.tokens("moe8_w4a8", t)
    ids, w = _oracle_route(x, "moe8_w4a8")
    out = _forward(lib, layer, x, ids, w, 1)
    rows = np.arange(t) if t <= 64 else np.sort(np.random.default_rng(4).choice(t, 48, replace=False))
    ref = ffn.moe_w4a8(_np(x)[rows], oe, ids[rows], w[rows])
    assert ffn.max_rel_l2(_np(out)[rows], ref) <= TOL_W4A8


@pytest.mark.parametrize("asym", [False, True], ids=["sym", "asym"])
def test_wide_bf16_prefill_tiles(lib, asym):
    """Enough 128-row tiles x 256-column blocks to take the wide bf16 prefill kernel
    (8 waves, 128 x 256 outputs) for both GEMMs (41 tiles x 8 column blocks each): 8
    experts, hidden 2048, inter 1024, top-2, T = 2048; a seeded sample of tokens against
    the oracle."""
    E, H, I, k, t = 8, 2048, 1024, 2, 2048
    make = random_expert_maker(107, H, I, sigma=0.03)
    layer = build_gpu_layer(lib, make, E, H, I, k, asym=asym)
    oe = OracleExperts(make, asym)
    x = synth.normal(synth.stream_key(108, t), (t, H), 1.0).to(torch.bfloat16)
    rng = np.random.default_rng(109)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(t)]).astype(np.int64)
    w = rng.dirichlet(np.ones(k), size=t)
    out = _forward(lib, layer, x, ids, w, 0)
    rows = np.sort(rng.choice(t, 40, replace=False))
    ref = ffn.moe_w4a16(_np(x)[rows], oe, ids[rows], w[rows])
    assert ffn.max_rel_l2(_np(out)[rows], ref) <= TOL_W4A16


# ------------------------------------------------------------------ single token: slot tiles
@pytest.mark.parametrize("mode", [0, 1], ids=["w4a16", "w4a8"])
@pytest.mark.parametrize("which", ["small_shared", "moe8"])
def test_single_token_slot_tiles_equal_permuted(lib, small, moe8, which, mode):
    """At t = 1 the forward takes one-row slot tiles straight from the routed ids (no
    permutation launch; on the 8-expert layer the down projection also splits K); the
    debug call runs the permuted path.  Each output row depends only on its own row and
    expert, so the two outputs agree bit for bit, and both match the oracle."""
    layer, oe = small if which == "small_shared" else moe8
    plan = lib.moe_int4_ffn_plan(layer, 1, mode)
    assert plan["slot_tiles"] and plan["kernel"] == "decode"
    for seed in range(3):
        x = synth.normal(synth.stream_key(71, seed), (1, layer.hidden), 1.0).to(torch.bfloat16)
        rng = np.random.default_rng(100 + seed)
        ids = rng.permutation(layer.num_experts)[: layer.top_k][None, :].astype(np.int32)
        w = rng.dirichlet(np.ones(layer.top_k))[None, :]
        out = _forward(lib, layer, x, ids, w, mode)
        dbg, _ = lib.moe_int4_ffn_debug(layer, x.cuda(), torch.as_tensor(ids).cuda(),
                                        torch.as_tensor(w, dtype=torch.float32).cuda(), mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(out.cpu(), dbg.cpu()), (which, mode, seed)
        shared = oe(layer.num_experts) if layer.shared else None
        fn = ffn.moe_w4a16 if mode == 0 else ffn.moe_w4a8
        ref = fn(_np(x), oe, ids, w, shared=shared) if shared is not None else fn(_np(x), oe, ids, w)
        assert ffn.max_rel_l2(_np(out), ref) <= (TOL_W4A16 if mode == 0 else TOL_W4A8)
