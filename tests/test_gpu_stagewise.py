"""Stage-by-stage parity of the MoE forward through moe_int4_ffn_debug.

Each stage of the GPU path is checked against the oracle applied to the GPU's own
inputs of that stage, so the bars can be tight:

* permutation: counts / offsets / perm / inv bit-exact;
* W4A8: x codes and scales bit-exact; h (fp32) within 2e-5 per row of the oracle's
  fp64 gate/up + SwiGLU on the same codes; the h codes and scales bit-exact against
  the oracle's fp32 quantisation of the GPU's own h; the down-projection INT32 group
  accumulators bit-exact on those codes; y within 2e-5 per row of the oracle's fp64
  rescale of them;
* W4A16: h (bf16) within 5e-3 per row of the fp64 h; y within 2e-5 per row of the
  oracle's down projection of the GPU's bf16 h;
* combine: the bf16 output within 4e-3 per row of the fp64 weighted sum of the GPU's
  per-position y (one bf16 rounding).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import ffn, permute as operm, router
from tests.helpers import OracleExperts, build_gpu_layer, random_expert_maker, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    require_gpu()
    import int4_group_quantized_g128_amd as lib
    return lib


def _np(t):
    return synth.to_numpy(t)


def _rows_rel(y, ref):
    """per-row relative L2 (zero reference rows need zero rows)"""
    return ffn.max_rel_l2(y, ref)


def check_stagewise(lib, layer, oe, x, ids, w, mode, shared):
    t, k = ids.shape
    E = layer.num_experts
    out, v = lib.moe_int4_ffn_debug(layer, x.cuda(), torch.as_tensor(ids, dtype=torch.int32).cuda(),
                                    torch.as_tensor(w, dtype=torch.float32).cuda(), mode=mode)
    torch.cuda.synchronize()
    S = v["slots_per_token"]
    assert S == k + (1 if shared else 0)
    # permutation over slots t * S + j (j == k: the shared expert)
    slot_ids = np.concatenate([ids, np.full((t, 1), E, np.int64)], axis=1) if shared else ids
    counts, offsets, perm, inv = operm.permute(slot_ids, E + (1 if shared else 0))
    assert np.array_equal(_np(v["counts"]), counts)
    assert np.array_equal(_np(v["offsets"]), offsets)
    assert np.array_equal(_np(v["perm"]), perm)
    assert np.array_equal(_np(v["inv"]), inv)
    x32 = _np(x).astype(np.float32)
    h = _np(v["h"]).astype(np.float64)
    y = _np(v["y"]).astype(np.float64)
    if mode == 1:
        qx, sx = ffn.act_quant_int8(x32)
        assert np.array_equal(_np(v["q_x"]), qx)
        assert np.array_equal(_np(v["s_x"]).view(np.uint32), sx.view(np.uint32))
        qh_gpu, sh_gpu = _np(v["q_h"]), _np(v["s_h"])
        qh_ref, sh_ref = ffn.act_quant_int8(_np(v["h"]))
        assert np.array_equal(qh_gpu, qh_ref)
        assert np.array_equal(sh_gpu.view(np.uint32), sh_ref.view(np.uint32))
    for e in range(E + (1 if shared else 0)):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        toks = perm[lo:hi] // S
        gate, up, down = oe(e)
        if mode == 1:
            g = ffn.linear_w4a8(qx[toks], sx[toks], gate)
            u = ffn.linear_w4a8(qx[toks], sx[toks], up)
            assert _rows_rel(h[lo:hi], ffn.silu(g) * u) <= 2e-5, f"h, expert {e}"
            # down-projection INT32 accumulators on the GPU's own h codes
            wdev = (layer.down[e * layer.dn_bytes:(e + 1) * layer.dn_bytes] if e < E else layer.shared_down)
            acc = lib.int4_w4a8_group_acc(v["q_h"][lo:hi].contiguous(), wdev, layer.hidden, layer.asymmetric)
            torch.cuda.synchronize()
            assert np.array_equal(_np(acc), ffn.group_acc(qh_gpu[lo:hi], ffn.widen_int8(down))), f"acc, expert {e}"
            y_ref = ffn.linear_w4a8(qh_gpu[lo:hi], sh_gpu[lo:hi], down)
        else:
            g = ffn.linear_w4a16(x32[toks], gate)
            u = ffn.linear_w4a16(x32[toks], up)
            assert _rows_rel(h[lo:hi], ffn.silu(g) * u) <= 5e-3, f"h, expert {e}"
            y_ref = ffn.linear_w4a16(h[lo:hi], down)
        assert _rows_rel(y[lo:hi], y_ref) <= 2e-5, f"y, expert {e}"
    # combine of the GPU's per-position outputs
    ref = np.zeros((t, layer.hidden))
    for tok in range(t):
        for j in range(k):
            ref[tok] += w[tok, j] * y[inv[tok * S + j]]
        if shared:
            ref[tok] += y[inv[tok * S + k]]
    assert _rows_rel(_np(out), ref) <= 4e-3


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
