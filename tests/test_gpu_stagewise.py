"""Stage-by-stage parity of the MoE forward through moe_int4_ffn_debug.

Each stage of the GPU path is checked against the oracle applied to the GPU's own
inputs of that stage, so the bars can be tight:

* permutation: counts / offsets / perm / inv bit-exact;
* W4A8: x codes and scales bit-exact; h (fp32) within 2e-5 per row of the oracle's
  fp64 gate/up + SwiGLU on the same codes; the h codes and scales bit-exact against
  the oracle's fp32 quantisation of the GPU's own h; the down-projection INT32 group
  accumulators bit-exact on those codes; y within 2e-5 per row of the oracle's fp64
  rescale of them;
* W4A16: h (bf16) within 5e-3 per row of the fp64 h; y within 1e-4 per row of the
  oracle's down projection of the GPU's bf16 h (the offset-widened weights are summed
  in fp32; tests/stagewise.py derives the bar);
* gate and up before SwiGLU, through the same GEMM core on the layer's own gate/up
  block: the INT32 group accumulators bit-exact on the GPU's x codes (W4A8), the fp32
  products within 1e-4 per row of the fp64 ones (W4A16);
* where the forward splits the down projection's K over workgroups (narrow layers at
  small batches), every K slice of y against the oracle's down projection restricted
  to that slice's groups, and their in-order sum as above;
* combine: the bf16 output within 4e-3 per row of the fp64 weighted sum of the GPU's
  per-position y (one bf16 rounding).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import router
from tests.helpers import OracleExperts, build_gpu_layer, random_expert_maker, require_gpu
from tests.stagewise import _np, check_stagewise

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    require_gpu()
    import int4_group_quantized_g128_amd as lib
    return lib


@pytest.fixture(scope="module")
def moe8(lib):
    cfg = synth.CONFIGS["moe8"]
    make = lambda e, device="cpu": synth.expert_weights("moe8", e, device)
    layer = build_gpu_layer(lib, make, cfg["experts"], cfg["hidden"], cfg["inter"], cfg["top_k"])
    return layer, OracleExperts(make, False)


@pytest.mark.parametrize("mode,t", [(1, 40), (1, 2048), (0, 40), (0, 512)],
                         ids=["w4a8-decode", "w4a8-prefill", "w4a16-decode", "w4a16-prefill"])
def test_moe8_stagewise(lib, moe8, mode, t):
    layer, oe = moe8
    name = "moe8_w4a8" if mode == 1 else "moe8"
    x = synth.tokens(name, t)
    wr, b = synth.router_weights(name)
    _, ids, w = router.route(_np(x), _np(wr), _np(b) if b is not None else None, synth.CONFIGS[name]["top_k"])
    check_stagewise(lib, layer, oe, x, ids, w, mode, shared=False)


@pytest.fixture(scope="module", params=[False, True], ids=["sym", "asym"])
def small_shared(lib, request):
    asym = request.param
    make = random_expert_maker(41 + asym, 256, 128)
    layer = build_gpu_layer(lib, make, 16, 256, 128, 4, asym=asym, shared=True)
    return layer, OracleExperts(make, asym)


@pytest.mark.parametrize("mode", [0, 1], ids=["w4a16", "w4a8"])
@pytest.mark.parametrize("t", [7, 300])
def test_shared_layer_stagewise(lib, small_shared, mode, t):
    layer, oe = small_shared
    x = synth.normal(synth.stream_key(42, t), (t, 256), 1.0).to(torch.bfloat16)
    rng = np.random.default_rng(t + 5)
    ids = np.stack([rng.permutation(16)[:4] for _ in range(t)]).astype(np.int64)
    w = rng.dirichlet(np.ones(4), size=t)
    check_stagewise(lib, layer, oe, x, ids, w, mode, shared=True)


@pytest.mark.parametrize("mode,t,ksplit", [(1, 1, 4), (0, 1, 4), (1, 2, 2), (0, 2, 2)],
                         ids=["w4a8-T1", "w4a16-T1", "w4a8-T2", "w4a16-T2"])
def test_moe8_stagewise_ksplit(lib, moe8, mode, t, ksplit):
    """The 8-expert layer at T = 1 and 2: the down projection splits K (4 and 2 slices)."""
    layer, oe = moe8
    x = synth.tokens("moe8", t)
    wr, _ = synth.router_weights("moe8")
    _, ids, w = router.route(_np(x), _np(wr), None, 2)
    check_stagewise(lib, layer, oe, x, ids, w, mode, shared=False, expect_ksplit=ksplit)


@pytest.fixture(scope="module")
def dense(lib):
    """The 2048/8192 dense SwiGLU FFN (asymmetric) as a one-expert layer."""
    cfg = synth.CONFIGS["dense"]
    g, u, d = synth.dense_ffn_weights("dense")
    layer = lib.MoELayer(1, cfg["hidden"], cfg["inter"], 1, asymmetric=True)
    layer.set_expert(0, g.cuda(), u.cuda(), d.cuda())
    torch.cuda.synchronize()
    return layer, OracleExperts(lambda e: (g, u, d), True)


@pytest.mark.parametrize("mode,t,ksplit", [(0, 1, 8), (1, 1, 8), (0, 4, 8), (0, 16, 8)],
                         ids=["w4a16-T1", "w4a8-T1", "w4a16-T4", "w4a16-T16"])
def test_dense_stagewise_ksplit(lib, dense, mode, t, ksplit):
    """Dense T = 1 / 4 / 16: 64 work items of two column blocks, so the down projection
    (K = 8192) splits into 8 slices that the combine adds in order."""
    layer, oe = dense
    x = synth.tokens("dense", t)
    ids = np.zeros((t, 1), np.int64)
    w = np.ones((t, 1))
    check_stagewise(lib, layer, oe, x, ids, w, mode, shared=False, expect_ksplit=ksplit)


@pytest.fixture(scope="module")
def wide(lib):
    """300 routed experts + a shared one on a small hidden size."""
    make = random_expert_maker(43, 128, 128)
    layer = build_gpu_layer(lib, make, 300, 128, 128, 8, shared=True)
    return layer, OracleExperts(make, False)


@pytest.mark.parametrize("mode", [0, 1], ids=["w4a16", "w4a8"])
@pytest.mark.parametrize("t", [1100, 2300])
def test_many_experts_large_batch_stagewise(lib, wide, mode, t):
    """9 t slots (9900 and 20700) take the many-workgroup permutation (ranges of 2048
    slots, the last one ragged): counts, offsets, perm and inv bit-exact through the
    forward, and the stages of a hot expert (a quarter of the tokens, many tiles), two
    ordinary ones and the shared expert."""
    layer, oe = wide
    x = synth.normal(synth.stream_key(44, t), (t, 128), 1.0).to(torch.bfloat16)
    rng = np.random.default_rng(t + 9)
    others = np.delete(np.arange(300), 7)
    ids = np.stack([np.concatenate([[7], rng.permutation(others)[:7]]) if i < t // 4 else rng.permutation(300)[:8]
                    for i in range(t)]).astype(np.int64)
    w = rng.dirichlet(np.ones(8), size=t)
    check_stagewise(lib, layer, oe, x, ids, w, mode, shared=True, experts=[7, 100, 299, 300])
