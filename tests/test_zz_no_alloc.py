"""The allocation-free forward (moe_int4_ffn_forward_noalloc, workspace in the library's
fixed per-GPU scratch array) against moe_int4_ffn_forward with a caller workspace:
bit-identical outputs (the same kernels), on consecutive calls whose second batch is
smaller than the first, through the C ABI; batches that need more than the scratch
size are refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from tests.helpers import build_gpu_layer, random_expert_maker, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    require_gpu()
    import int4_group_quantized_g128_amd as lib
    return lib


def _batch(t, E, k, H, seed):
    x = synth.normal(synth.stream_key(seed, t), (t, H), 1.0).to(torch.bfloat16).cuda()
    rng = np.random.default_rng(seed + t)
    ids = torch.as_tensor(np.stack([rng.permutation(E)[:k] for _ in range(t)]), dtype=torch.int32).cuda()
    w = torch.as_tensor(rng.dirichlet(np.ones(k), size=t), dtype=torch.float32).cuda()
    return x, ids, w


def _noalloc_raw(lib, layer, x, ids, w, mode):
    """Through the raw C entry point (no workspace argument)."""
    out = torch.full_like(x, float("nan"))
    rc = lib._lib.raw.moe_int4_ffn_forward_noalloc(ctypes.byref(layer.desc), ctypes.c_void_p(x.data_ptr()), x.shape[0],
                                                   ctypes.c_void_p(ids.data_ptr()), ctypes.c_void_p(w.data_ptr()), mode,
                                                   ctypes.c_void_p(out.data_ptr()),
                                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, lib._lib.raw.q4_last_error()
    return out


@pytest.fixture(scope="module")
def small_shared(lib):
    make = random_expert_maker(61, 256, 128)
    return build_gpu_layer(lib, make, 16, 256, 128, 4, shared=True)


@pytest.mark.parametrize("mode", [0, 1], ids=["w4a16", "w4a8"])
def test_noalloc_equals_forward_two_calls(lib, small_shared, mode):
    layer = small_shared
    for t in (300, 7):       # the second call smaller than the first
        x, ids, w = _batch(t, 16, 4, 256, 62)
        ref = lib.moe_int4_ffn_forward(layer, x, ids, w, mode=mode)
        got = _noalloc_raw(lib, layer, x, ids, w, mode)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"t={t}"


@pytest.fixture(scope="module")
def moe8(lib):
    cfg = synth.CONFIGS["moe8"]
    make = lambda e, device="cpu": synth.expert_weights("moe8", e, device)
    return build_gpu_layer(lib, make, cfg["experts"], cfg["hidden"], cfg["inter"], cfg["top_k"])


def test_noalloc_moe8_prefill_then_split_decode(lib, moe8):
    """The 8-expert layer: T = 512 (prefill tiles) then T = 1 (the down projection split
    over K slices), both against the workspace forward."""
    for t, mode in ((512, 1), (1, 1), (256, 0), (1, 0)):
        x, ids, w = _batch(t, 8, 2, 2048, 63)
        ref = lib.moe_int4_ffn_forward(moe8, x, ids, w, mode=mode)
        got = lib.moe_int4_ffn_forward_noalloc(moe8, x, ids, w, mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), (t, mode)


def test_noalloc_many_workgroup_permutation(lib):
    """300 routed experts + a shared one (hidden 128): T = 1100 is 9900 routed slots, so
    the permutation runs over many workgroups with its per-range counts in the scratch
    array; then T = 40 (one workgroup)."""
    layer = build_gpu_layer(lib, random_expert_maker(64, 128, 128), 300, 128, 128, 8, shared=True)
    for t, mode in ((1100, 1), (40, 1), (1100, 0)):
        x, ids, w = _batch(t, 300, 8, 128, 65)
        ref = lib.moe_int4_ffn_forward(layer, x, ids, w, mode=mode)
        got = _noalloc_raw(lib, layer, x, ids, w, mode)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), (t, mode)


def test_noalloc_refuses_batches_beyond_the_scratch(lib, moe8):
    t = 1
    while lib.moe_int4_ffn_plan(moe8, t, 0)["workspace_bytes"] <= lib.Q4_NOALLOC_SCRATCH_BYTES:
        t *= 2
    x, ids, w = _batch(t, 8, 2, 2048, 64)
    with pytest.raises(lib.Q4Error) as e:
        lib.moe_int4_ffn_forward_noalloc(moe8, x, ids, w, mode=0)
    assert e.value.code == 5      # Q4_ERR_WORKSPACE, before any launch
    torch.cuda.synchronize()
