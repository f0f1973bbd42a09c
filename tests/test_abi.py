"""The C ABI loads, exports every declared symbol and rejects bad arguments on the
host before any launch (CPU only: no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4moe.h")


@pytest.fixture(scope="module")
def L():
    from int4_group_quantized_g128_amd import _lib
    return _lib


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"Q4_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("quantize_int4_g128", "moe_route_topk", "moe_int4_ffn_forward"):
        assert required in names
    assert len(names) == len(set(names))


def test_library_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L.raw, n), n


def test_status_strings_and_version(L):
    assert L.raw.q4_status_string(0) == b"ok"
    for c in range(1, 8):
        assert L.raw.q4_status_string(c) not in (b"", b"unknown status")
    assert L.raw.q4_status_string(99) == b"unknown status"
    assert b"gfx950" in L.raw.q4_version()


def _err(L):
    return L.raw.q4_last_error().decode()


def test_quantize_validation(L):
    r = L.raw
    fake = ctypes.c_void_p(4096)
    assert r.quantize_int4_g128(fake, 9, 16, 128, 0, fake, fake, None, None, None) == L.Q4_ERR_DTYPE
    assert r.quantize_int4_g128(fake, 0, 16, 100, 0, fake, fake, None, None, None) == L.Q4_ERR_SHAPE
    assert "128" in _err(L)
    assert r.quantize_int4_g128(fake, 0, 0, 128, 0, fake, fake, None, None, None) == L.Q4_ERR_SHAPE
    assert r.quantize_int4_g128(None, 0, 16, 128, 0, fake, fake, None, None, None) == L.Q4_ERR_NULL
    assert r.quantize_int4_g128(fake, 0, 16, 128, 1, fake, fake, None, None, None) == L.Q4_ERR_NULL
    assert r.quantize_int4_g128(fake, 0, 16, 128, 0, fake, fake, fake, None, None) == L.Q4_ERR_NULL
    assert r.quantize_int4_g128(ctypes.c_void_p(4100), 0, 16, 128, 0, fake, fake, None, None, None) == L.Q4_ERR_ALIGN


def test_repack_validation(L):
    r = L.raw
    fake = ctypes.c_void_p(4096)
    need = r.q4_device_bytes(64, 256, 0)
    assert need == 64 * 128 + 2 * 64 * 2 + (256 - (2 * 64 * 2) % 256) % 256
    assert r.q4_device_bytes(40, 256, 0) == 0 and r.q4_device_bytes(64, 200, 0) == 0
    assert r.q4_device_bytes(64, 256, 1) == need + 256
    assert r.q4_repack_device(fake, fake, None, 64, 256, 0, 0, fake, need - 1, None) == L.Q4_ERR_WORKSPACE
    assert r.q4_repack_device(fake, fake, None, 48, 256, 0, 1, fake, need, None) == L.Q4_ERR_SHAPE
    assert r.q4_repack_device(fake, fake, None, 64, 256, 1, 0, fake, need * 2, None) == L.Q4_ERR_NULL
    assert r.q4_repack_device(fake, fake, None, 64, 256, 0, 7, fake, need, None) == L.Q4_ERR_DTYPE


def test_route_validation(L):
    r = L.raw
    fake = ctypes.c_void_p(4096)
    assert r.moe_route_topk(fake, fake, None, 4, 256, 8, 9, fake, fake, fake, fake, 1 << 30, None) == L.Q4_ERR_SHAPE
    assert r.moe_route_topk(fake, fake, None, 4, 256, 2000, 2, fake, fake, fake, fake, 1 << 30, None) == L.Q4_ERR_SHAPE
    assert r.moe_route_topk(fake, fake, None, 4, 250, 8, 2, fake, fake, fake, fake, 1 << 30, None) == L.Q4_ERR_SHAPE
    assert r.moe_route_topk(fake, fake, None, 4, 256, 8, 2, None, fake, fake, fake, 1 << 30, None) == L.Q4_ERR_NULL
    need = r.moe_route_workspace_bytes(4, 256, 8)
    assert need > 0
    assert r.moe_route_topk(fake, fake, None, 4, 256, 8, 2, fake, fake, fake, fake, need - 1, None) == L.Q4_ERR_WORKSPACE
    odd = ctypes.c_void_p(4096 + 4)
    assert r.moe_route_topk(fake, fake, None, 4, 256, 8, 2, fake, fake, fake, odd, need, None) == L.Q4_ERR_ALIGN
    # from 512 tokens and 64 experts the workspace also holds the three bf16 parts of the weights
    big = r.moe_route_workspace_bytes(512, 256, 64)
    assert big >= 3 * 64 * 256 * 2 + 512 * 64 * 4
    # t == 0 is a successful no-op, even without buffers
    assert r.moe_route_topk(None, None, None, 0, 256, 8, 2, None, None, None, None, 0, None) == L.Q4_OK


def test_permute_and_act_quant_validation(L):
    r = L.raw
    fake = ctypes.c_void_p(4096)
    assert r.moe_permute(fake, 4, 3, 2, fake, fake, fake, fake, None) == L.Q4_ERR_SHAPE
    assert r.moe_permute(fake, 4, 1, 5000, fake, fake, fake, fake, None) == L.Q4_ERR_SHAPE
    assert r.moe_permute(fake, 4, 1, 8, None, fake, fake, fake, None) == L.Q4_ERR_NULL
    assert r.act_quant_int8(fake, L.Q4_F16, 4, 128, fake, fake, None) == L.Q4_ERR_DTYPE
    assert r.act_quant_int8(fake, L.Q4_BF16, 4, 100, fake, fake, None) == L.Q4_ERR_SHAPE
    assert r.act_quant_int8(None, L.Q4_BF16, 0, 128, None, None, None) == L.Q4_OK


def _layer(L, **kw):
    d = dict(num_experts=8, hidden=256, inter=128, top_k=2, asymmetric=0, shared_inter=0,
             gate_up=4096, down=8192, shared_gate_up=None, shared_down=None)
    d.update(kw)
    return L.Q4MoELayer(**d)


def test_forward_validation(L):
    r = L.raw
    fake = ctypes.c_void_p(4096)
    ok = _layer(L)
    need = r.moe_int4_ffn_workspace_bytes(ctypes.byref(ok), 10, 0)
    assert need > 0
    assert r.moe_int4_ffn_workspace_bytes(ctypes.byref(ok), 10, 1) > need
    call = lambda lay, t=10, mode=0, ws=need, x=fake: r.moe_int4_ffn_forward(
        ctypes.byref(lay), x, t, fake, fake, mode, fake, fake, ws, None)
    assert call(ok, ws=need - 1) == L.Q4_ERR_WORKSPACE
    assert call(ok, mode=5) == L.Q4_ERR_DTYPE
    assert call(_layer(L, top_k=9)) == L.Q4_ERR_SHAPE
    assert call(_layer(L, hidden=200)) == L.Q4_ERR_SHAPE
    assert call(_layer(L, inter=100)) == L.Q4_ERR_SHAPE
    assert call(_layer(L, gate_up=None)) == L.Q4_ERR_NULL
    assert call(_layer(L, down=8200)) == L.Q4_ERR_ALIGN
    assert call(_layer(L, shared_inter=256, shared_gate_up=4096, shared_down=4096)) == L.Q4_ERR_UNSUPPORTED
    assert call(_layer(L, shared_inter=128)) == L.Q4_ERR_NULL
    assert call(ok, x=ctypes.c_void_p(4098)) == L.Q4_ERR_ALIGN
    assert call(ok, x=None) == L.Q4_ERR_NULL
    assert call(ok, t=-1) == L.Q4_ERR_SHAPE
    assert call(ok, t=0, x=None) == L.Q4_OK
    assert r.moe_int4_ffn_workspace_bytes(None, 10, 0) == 0


def test_forward_workspace_sizes(L):
    """Host sizing only: zero tokens, and the K-split partial slices of y that narrow
    decode layers get (a one-expert 2048/8192 FFN at t = 1: eight slices of 2048 fp32)."""
    r = L.raw
    for mode in (0, 1):
        assert r.moe_int4_ffn_workspace_bytes(ctypes.byref(_layer(L)), 0, mode) >= 0
    dense = _layer(L, num_experts=1, top_k=1, hidden=2048, inter=8192)
    need = r.moe_int4_ffn_workspace_bytes(ctypes.byref(dense), 1, 0)
    assert need >= 8 * 2048 * 4 + 8192 * 2
    wide = _layer(L, num_experts=256, top_k=8, hidden=7168, inter=2048)
    # 64 tokens: enough work items, one slice (y of 512 positions x 7168 fp32)
    assert r.moe_int4_ffn_workspace_bytes(ctypes.byref(wide), 64, 0) < 2 * 512 * 7168 * 4 + 512 * 2048 * 2 + (1 << 20)


def test_linear_and_group_acc_validation(L):
    r = L.raw
    fake = ctypes.c_void_p(4096)
    assert r.int4_linear_forward(fake, L.Q4_F32, 4, 128, fake, 64, 0, fake, None) == L.Q4_ERR_DTYPE
    assert r.int4_linear_forward(fake, L.Q4_F16, 4, 128, fake, 48, 0, fake, None) == L.Q4_ERR_SHAPE
    assert r.int4_linear_forward(fake, L.Q4_F16, 4, 128, None, 64, 0, fake, None) == L.Q4_ERR_NULL
    assert r.int4_w4a8_group_acc(fake, 4, 130, fake, 64, 0, fake, None) == L.Q4_ERR_SHAPE
    assert r.int4_w4a8_group_acc(fake, 0, 128, fake, 64, 0, fake, None) == L.Q4_OK


def test_binding_refuses_cpu_tensors(L):
    import torch
    with pytest.raises(ValueError):
        L.quantize_int4_g128(torch.zeros((16, 128)))


def test_expert_bits_by_hotness_matches_the_oracle_rule(L):
    import numpy as np
    from oracle import ffn
    rng = np.random.default_rng(5)
    for E, frac, shared in ((256, 0.05, False), (8, 0.25, True), (17, 0.0, False), (9, 1.0, True), (64, 0.1, False)):
        counts = rng.integers(0, 6, E)
        assert L.expert_bits_by_hotness(counts.tolist(), frac, shared) == ffn.bits_by_hotness(counts, frac, shared)
    with pytest.raises(L.Q4Error):
        L.expert_bits_by_hotness([1, 2], 1.5)
    with pytest.raises(L.Q4Error):
        L.expert_bits_by_hotness([1, -2], 0.5)
    # the raw C entry point, host arrays only
    counts = (ctypes.c_int64 * 4)(3, 9, 9, 1)
    out = (ctypes.c_int32 * 5)()
    assert L.raw.moe_expert_bits_by_hotness(counts, 4, 0.5, 1, out) == L.Q4_OK
    assert list(out) == [4, 8, 8, 4, 8]      # ties: the lower index first; shared 8
    assert L.raw.moe_expert_bits_by_hotness(counts, 4, 0.25, 0, out) == L.Q4_OK
    assert list(out)[:4] == [4, 8, 4, 4]
    assert L.raw.moe_expert_bits_by_hotness(None, 4, 0.25, 0, out) == L.Q4_ERR_NULL
    assert L.raw.moe_expert_bits_by_hotness(counts, 0, 0.25, 0, out) == L.Q4_ERR_SHAPE


def test_mixed_layer_validation(L):
    r = L.raw
    fake = ctypes.c_void_p(4096)
    desc = L.Q4MoELayer(8, 256, 128, 2, 0, 0, 4096, 4096, None, None, 0, 4096, 4096, 4096)
    # mixed layers run with INT8 activations only
    assert r.moe_int4_ffn_workspace_bytes(ctypes.byref(desc), 4, L.Q4_W4A16) == 0
    assert r.moe_int4_ffn_workspace_bytes(ctypes.byref(desc), 4, L.Q4_W4A8) > 0
    for bad in (dict(asymmetric=1), dict(weight_bits=8), dict(down_offsets=None)):
        d = L.Q4MoELayer(8, 256, 128, 2, 0, 0, 4096, 4096, None, None, 0, 4096, 4096, 4096)
        for key, v in bad.items():
            setattr(d, key, v)
        assert r.moe_int4_ffn_workspace_bytes(ctypes.byref(d), 4, L.Q4_W4A8) == 0
    assert r.moe_int4_ffn_forward(ctypes.byref(desc), fake, 4, fake, fake, L.Q4_W4A16, fake, fake, 1 << 20,
                                  None) == L.Q4_ERR_DTYPE


def test_grouped_format_sizes_and_validation(L):
    from oracle import layout
    r = L.raw
    for n, k, asym, g in ((64, 512, 0, 32), (64, 512, 0, 64), (32, 256, 0, 128), (96, 1024, 0, 256),
                          (96, 1024, 1, 256), (64, 512, 1, 128)):
        assert r.q4_device_bytes_grouped(n, k, asym, g) == layout.device_bytes(n, k, bool(asym), g)
    assert r.q4_device_bytes_grouped(64, 512, 0, 128) == r.q4_device_bytes(64, 512, 0)
    assert r.q4_device_bytes_grouped(64, 512, 1, 32) == 0      # zero points need groups >= 128
    assert r.q4_device_bytes_grouped(64, 384, 0, 256) == 0     # k % group
    assert r.q4_device_bytes_grouped(64, 512, 0, 48) == 0
    fake = ctypes.c_void_p(4096)
    assert r.quantize_int4_grouped(fake, L.Q4_F32, 4, 256, 48, 0, fake, fake, None, None, None) == L.Q4_ERR_SHAPE
    assert r.quantize_int4_grouped(fake, L.Q4_F32, 4, 256, 32, 1, fake, fake, fake, None, None) == \
        L.Q4_ERR_UNSUPPORTED
    assert r.quantize_int4_grouped(fake, L.Q4_F32, 4, 384, 256, 0, fake, fake, None, None, None) == L.Q4_ERR_SHAPE
    assert r.q4_repack_device_grouped(fake, fake, None, 64, 512, 0, 32, L.Q4_REPACK_PLAIN, fake, 16, None) == \
        L.Q4_ERR_WORKSPACE


def test_expert_groups_by_hotness_matches_the_oracle_rule(L):
    import numpy as np
    from oracle import ffn
    rng = np.random.default_rng(6)
    for E, shared in ((256, False), (8, True), (17, False), (64, True)):
        counts = rng.integers(0, 50, E)
        counts[rng.integers(0, E)] = 0
        assert L.expert_groups_by_hotness(counts.tolist(), 0.05, 0.1, shared) == \
            ffn.groups_by_hotness(counts, 0.05, 0.1, shared)
    # hand case: total 100 over 4 experts, even share 25, cold below 2.5 -> 256
    counts = (ctypes.c_int64 * 4)(2, 60, 35, 3)
    out = (ctypes.c_int32 * 5)()
    assert L.raw.moe_expert_groups_by_hotness(counts, 4, 0.25, 0.1, 1, out) == L.Q4_OK
    assert list(out) == [256, 32, 64, 64, 32]
    with pytest.raises(L.Q4Error):
        L.expert_groups_by_hotness([1, 2], 0.05, -1.0)


def test_grouped_layer_validation(L):
    r = L.raw

    def desc(**kw):
        d = L.Q4MoELayer(8, 256, 256, 2, 0, 0, 4096, 4096, None, None, 0, None, 4096, 4096, 4096)
        for key, v in kw.items():
            setattr(d, key, v)
        return d
    for mode in (L.Q4_W4A16, L.Q4_W4A8):
        assert r.moe_int4_ffn_workspace_bytes(ctypes.byref(desc()), 300, mode) > 0
    assert r.moe_int4_ffn_workspace_bytes(ctypes.byref(desc()), 4, L.Q4_W8A8) == 0
    assert r.moe_int4_ffn_workspace_bytes(ctypes.byref(desc(expert_bits=4096)), 4, L.Q4_W4A16) == 0
    for bad in (dict(asymmetric=1), dict(weight_bits=8), dict(gate_up_offsets=None)):
        assert r.moe_int4_ffn_workspace_bytes(ctypes.byref(desc(**bad)), 4, L.Q4_W4A16) == 0


def _plan_desc(L, E, H, I, k, shared=False, asym=0, **kw):
    d = L.Q4MoELayer(E, H, I, k, asym, I if shared else 0, 4096, 4096, 4096 if shared else None,
                     4096 if shared else None, 0, None, None, None, None)
    for key, v in kw.items():
        setattr(d, key, v)
    return d


def test_plan_kernel_choice(L):
    """Host-only plan query: which GEMM kernel and tiles the forward takes (no GPU)."""
    moe256 = _plan_desc(L, 256, 7168, 2048, 8, shared=True)
    moe8 = _plan_desc(L, 8, 2048, 1024, 2)
    dense = _plan_desc(L, 1, 2048, 8192, 1, asym=1)
    W16, W8 = L.Q4_W4A16, L.Q4_W4A8
    cases = [
        # (layer, t, mode) -> (kernel, tile rows, down K slices)
        ((moe256, 1, W16), ("decode", 16, 1)),
        ((moe256, 64, W16), ("decode", 16, 1)),
        ((moe256, 512, W16), ("decode", 16, 1)),      # 16 rows per expert, bf16: decode tiles
        ((moe256, 512, W8), ("prefill", 128, 1)),     # from 9 rows with INT8 activations
        ((moe256, 768, W16), ("prefill", 128, 1)),    # 24 rows, >= 2048 items
        ((moe256, 1280, W8), ("prefill", 128, 1)),
        ((moe256, 4096, W16), ("prefill", 128, 1)),
        ((moe8, 1, W16), ("decode", 16, 4)),          # narrow: the down projection splits K
        ((moe8, 2, W8), ("decode", 16, 2)),
        ((moe8, 40, W8), ("decode", 16, 1)),          # est. 512 items: no split
        ((moe8, 192, W16), ("decode", 64, 1)),        # 48 rows, few items: decode tiles
        ((moe8, 256, W8), ("prefill", 128, 1)),       # 64 rows per expert
        ((dense, 1, W16), ("decode", 16, 8)),
        ((dense, 16, W16), ("decode", 16, 8)),
        ((dense, 17, W16), ("decode", 32, 1)),
    ]
    for (desc, t, mode), (kernel, rows, ks) in cases:
        p = L.moe_int4_ffn_plan(desc, t, mode)
        assert (p["kernel"], p["tile_rows"], p["down_ksplit"]) == (kernel, rows, ks), (t, mode, p)
        assert p["workspace_bytes"] == L.raw.moe_int4_ffn_workspace_bytes(ctypes.byref(desc), t, mode)
        assert not p["prefill_addr_limited"]
        one = desc is dense and kernel == "decode"
        assert p["rows_in_token_order"] == one and p["combine_in_down"] == (one and ks == 1)
        # a single token on a one-format layer: one-row slot tiles, no permutation launch
        assert p["slot_tiles"] == (t == 1 and desc is not dense), (t, p)
    # layers with several weight formats keep the 64-rows-per-expert rule
    mixed = _plan_desc(L, 256, 7168, 2048, 8, shared=True, expert_bits=4096, gate_up_offsets=4096,
                       down_offsets=4096)
    assert L.moe_int4_ffn_plan(mixed, 1280, W8)["kernel"] == "decode"
    assert not L.moe_int4_ffn_plan(mixed, 1, W8)["slot_tiles"]   # formats: the permutation orders them
    assert L.moe_int4_ffn_plan(mixed, 2048, W8)["kernel"] == "prefill"
    grouped = _plan_desc(L, 256, 7168, 2048, 8, shared=True, expert_groups=4096, gate_up_offsets=4096,
                         down_offsets=4096)
    assert L.moe_int4_ffn_plan(grouped, 768, W16)["kernel"] == "decode"
    assert L.moe_int4_ffn_plan(grouped, 4096, W16)["kernel"] == "prefill"


def test_plan_no_empty_k_slice(L):
    """I = 1152 (9 groups): 4 slices of ceil(9/4) = 3 groups would leave the last one
    empty; the plan takes 3."""
    p = L.moe_int4_ffn_plan(_plan_desc(L, 8, 2048, 1152, 2), 1, L.Q4_W4A16)
    assert p["down_ksplit"] == 3


def test_plan_prefill_addressing_limit(L):
    """Past the prefill kernels' 32-bit activation offsets (h of the 256-expert W4A16 down
    projection passes 2^31 bytes at t * 9 * 2048 * 2 >= 2^31) the forward takes the
    decode kernel, which addresses with 64-bit offsets, and the plan says so."""
    moe256 = _plan_desc(L, 256, 7168, 2048, 8, shared=True)
    t_lim = (1 << 31) // (9 * 2048 * 2)
    p = L.moe_int4_ffn_plan(moe256, t_lim, L.Q4_W4A16)
    assert p["kernel"] == "prefill" and not p["prefill_addr_limited"]
    p = L.moe_int4_ffn_plan(moe256, t_lim + 1, L.Q4_W4A16)
    assert p["kernel"] == "decode" and p["prefill_addr_limited"]
    # INT8 activations: x codes are 1 byte, h codes 1 byte per element (limit at 2^31 / (9 * 2048))
    t8 = (1 << 31) // (9 * 2048)
    assert L.moe_int4_ffn_plan(moe256, t8 - 8, L.Q4_W4A8)["kernel"] == "prefill"
    assert L.moe_int4_ffn_plan(moe256, t8 + 8, L.Q4_W4A8)["prefill_addr_limited"]


def test_plan_validation(L):
    p = L.Q4FfnPlan()
    assert L.raw.moe_int4_ffn_plan(None, 4, L.Q4_W4A16, ctypes.byref(p)) == L.Q4_ERR_NULL
    d = _plan_desc(L, 8, 2048, 1024, 2)
    assert L.raw.moe_int4_ffn_plan(ctypes.byref(d), 4, L.Q4_W4A16, None) == L.Q4_ERR_NULL
    assert L.raw.moe_int4_ffn_plan(ctypes.byref(d), -1, L.Q4_W4A16, ctypes.byref(p)) == L.Q4_ERR_SHAPE
    assert L.raw.moe_int4_ffn_plan(ctypes.byref(d), 4, L.Q4_W8A8, ctypes.byref(p)) == L.Q4_ERR_DTYPE


def test_two_bit_format_sizes_and_apex_rule(L):
    import numpy as np
    from oracle import ffn, layout
    r = L.raw
    for n, k in ((64, 512), (32, 256), (96, 7168)):
        assert r.q2_device_bytes(n, k) == layout.device_bytes2(n, k)
    assert r.q2_device_bytes(24, 256) == 0 and r.q2_device_bytes(64, 200) == 0
    fake = ctypes.c_void_p(4096)
    assert r.quantize_int2_g128(fake, L.Q4_F32, 4, 200, fake, fake, None, None) == L.Q4_ERR_SHAPE
    assert r.quantize_int2_g128(fake, 9, 4, 256, fake, fake, None, None) == L.Q4_ERR_DTYPE
    assert r.q2_repack_device(fake, fake, 64, 512, L.Q4_REPACK_PLAIN, fake, 16, None) == L.Q4_ERR_WORKSPACE
    assert r.q2_repack_device(fake, fake, 48, 512, L.Q4_REPACK_GATE_UP, fake, 1 << 20, None) == L.Q4_ERR_SHAPE
    rng = np.random.default_rng(8)
    for E, frac8, cold, shared in ((256, 0.0, 0.25, True), (8, 0.25, 0.5, False), (17, 0.05, 1.0, True)):
        counts = rng.integers(0, 40, E)
        assert L.expert_bits_apex(counts.tolist(), frac8, cold, shared) == \
            [int(b) for b in ffn.bits_apex(counts, frac8, cold, shared)]
