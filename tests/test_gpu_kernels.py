"""GPU parity of the single-kernel entry points against the oracle (MI355X)."""
import numpy as np
import pytest
import torch

import synth
from oracle import ffn, layout, permute, quant, router
from tests.helpers import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    require_gpu()
    import int4_group_quantized_g128_amd as lib
    return lib


def _np(t):
    return synth.to_numpy(t)


def _special_weights(n, k, seed):
    w = synth.normal(synth.stream_key(seed, 77), (n, k), 0.02)
    w[0, :128] = 0.0                        # zero group
    w[1, :128] *= 1e-9                      # scale underflows binary16 -> 0
    w[2, 128:256] *= 1e-3                   # subnormal binary16 scale
    w[3, :128] *= 1e5                       # large scale (still finite in binary16)
    w[4, :128] = torch.abs(w[4, :128])      # all positive
    w[5, :128] = -torch.abs(w[5, :128])     # all negative
    return w


# ------------------------------------------------------------------ A1 quantise
@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("n,k", [(37, 384), (64, 2048)])
def test_quantize_bit_exact(lib, asym, dtype, n, k):
    w = _special_weights(n, k, 1).to(dtype)
    packed, scales, zeros = lib.quantize_int4_g128(w.cuda(), asymmetric=asym)
    rp, rs, rz = quant.quantize_pack(_np(w), asym)
    assert np.array_equal(_np(packed), rp)
    assert np.array_equal(_np(scales).view(np.uint16), rs)
    if asym:
        assert np.array_equal(_np(zeros), rz)


def test_quantize_linear_workload_bit_exact(lib):
    """The 2048 x 2048 linear workload with 0.1 % outliers x20, symmetric."""
    _, w = synth.linear_inputs()
    packed, scales, _ = lib.quantize_int4_g128(w.cuda())
    rp, rs, _ = quant.quantize_pack(_np(w), False)
    assert np.array_equal(_np(packed), rp)
    assert np.array_equal(_np(scales).view(np.uint16), rs)


def test_quantize_flags_nonfinite_and_overflow(lib):
    w = torch.zeros((16, 256))
    w[3, 5] = float("inf")
    w[7, 200] = 1e6                          # amax / 7 > 65504
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    lib.quantize_int4_g128(w.cuda(), flags=flags)
    assert int(flags.item()) == 3


# ------------------------------------------------------------------ A2 repack
@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("gate_up", [False, True])
def test_repack_bit_exact(lib, asym, gate_up):
    n, k = 96, 640
    w = _special_weights(n, k, 2)
    packed, scales, zeros = lib.quantize_int4_g128(w.cuda(), asymmetric=asym)
    dev = lib.q4_repack_device(packed, scales, zeros, n, k, asym, gate_up=gate_up)
    rp, rs, rz = quant.quantize_pack(_np(w), asym)
    ref = layout.to_device(rp, rs, rz, n, k, asym, gate_up)
    assert np.array_equal(_np(dev), ref)


# ------------------------------------------------------------------ A3/A4 router
def _router_case(name, t, salt=0):
    x = synth.tokens(name, t, salt=salt)
    w, b = synth.router_weights(name)
    return x, w, b


@pytest.mark.parametrize("name,t", [("moe8", 1), ("moe8", 37), ("moe8", 256), ("moe256", 1),
                                    ("moe256", 64), ("moe256", 300)])
def test_router_parity(lib, name, t):
    cfg = synth.CONFIGS[name]
    x, w, b = _router_case(name, t)
    logits, ids, wts = lib.moe_route_topk(x.cuda(), w.cuda(), b.cuda() if b is not None else None, cfg["top_k"])
    L64 = router.logits_fp64(_np(x), _np(w), _np(b) if b is not None else None)
    Lg = _np(logits)
    # fp32 accumulation error bound: a few ulps of sum |x| |w| per logit
    mag = np.abs(_np(x)).astype(np.float64) @ np.abs(_np(w)).astype(np.float64).T
    assert np.all(np.abs(Lg - L64) <= 2e-6 * mag + 1e-6)
    # selection is bit-exact given the GPU's own fp32 logits
    ref_ids = router.select_topk(Lg, cfg["top_k"])
    assert np.array_equal(_np(ids), ref_ids)
    ref_w = router.topk_weights(Lg, ref_ids)
    assert np.allclose(_np(wts), ref_w, rtol=2e-6, atol=1e-7)
    assert np.allclose(_np(wts).sum(axis=1), 1.0, atol=2e-6)


@pytest.mark.parametrize("name,t", [("moe256", 1), ("moe256", 64), ("moe8", 37)])
def test_router_workspace_contents_do_not_matter(lib, name, t):
    """The router's workspace needs no initial contents: a workspace of 0xFF bytes or of
    zeros, and the same workspace again (what the previous call left behind), give the
    same logits, ids and weights, bit for bit."""
    cfg = synth.CONFIGS[name]
    x, w, b = _router_case(name, t, salt=3)
    x, w, b = x.cuda(), w.cuda(), (b.cuda() if b is not None else None)
    k, e, h = cfg["top_k"], w.shape[0], x.shape[1]
    L = lib._lib
    nbytes = int(L.raw.moe_route_workspace_bytes(t, h, e))
    outs = []
    for fill in (0xFF, None, 0x00, None):
        if fill is not None:
            ws = torch.full((max(nbytes, 1),), fill, dtype=torch.uint8, device="cuda")
        logits = torch.empty((t, e), dtype=torch.float32, device="cuda")
        ids = torch.empty((t, k), dtype=torch.int32, device="cuda")
        wts = torch.empty((t, k), dtype=torch.float32, device="cuda")
        rc = L.raw.moe_route_topk(L._ptr(x), L._ptr(w), L._ptr(b), t, h, e, k, L._ptr(logits), L._ptr(ids),
                                  L._ptr(wts), L._ptr(ws), nbytes, L._stream())
        assert rc == 0
        torch.cuda.synchronize()
        outs.append((logits.cpu(), ids.cpu(), wts.cpu()))
    ref = lib.moe_route_topk(x, w, b, k)
    for o in outs:
        for a, r in zip(o, ref):
            assert torch.equal(a, r.cpu())


@pytest.mark.parametrize("t,h,e,k", [(17, 512, 100, 3), (9, 256, 1000, 70), (3, 768, 64, 64), (40, 256, 300, 8),
                                     (600, 512, 256, 8), (517, 256, 100, 5), (2100, 256, 130, 4),
                                     (520, 272, 64, 2), (2050, 784, 72, 6), (100, 512, 256, 8),
                                     (130, 256, 64, 2), (200, 768, 72, 6), (511, 256, 80, 4)])
def test_router_parity_shapes(lib, t, h, e, k):
    """Expert counts across the one-, two-, four-, eight- and sixteen-slot variants of
    the selection kernel, k up to e and beyond one wave's width; batches of 512 and 2048
    tokens and more take the 32 x 64- and 64 x 64-tile split-weight logit kernels (ragged
    in tokens and experts here, and with hidden sizes that end in half a 32-wide K step);
    from 65 tokens (64 experts or more) the small-batch logit kernel takes 32- and then
    64-token tiles (ragged in tokens and experts here)."""
    x = synth.normal(synth.stream_key(70, t, e), (t, h), 1.0).to(torch.bfloat16)
    w = synth.normal(synth.stream_key(71, h, e), (e, h), 0.05)
    b = synth.normal(synth.stream_key(72, e), (e,), 0.3)
    logits, ids, wts = lib.moe_route_topk(x.cuda(), w.cuda(), b.cuda(), k)
    Lg = _np(logits)
    L64 = router.logits_fp64(_np(x), _np(w), _np(b))
    mag = np.abs(_np(x)).astype(np.float64) @ np.abs(_np(w)).astype(np.float64).T
    assert np.all(np.abs(Lg - L64) <= 2e-6 * mag + 1e-6)
    ref_ids = router.select_topk(Lg, k)
    assert np.array_equal(_np(ids), ref_ids)
    assert np.allclose(_np(wts), router.topk_weights(Lg, ref_ids), rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("t", [5, 600])
def test_router_nonfinite_weight(lib, t):
    """A non-finite router weight on both logit kernels (fp32 matrix cores below 512
    tokens, the three-part bf16 split from 512): +inf times positive x gives a +inf logit,
    so that expert is every token's first choice, a NaN weight a NaN logit, and the other
    logits keep the fp32 bound."""
    e, h, k = 64, 256, 4
    x = synth.normal(synth.stream_key(73, t), (t, h), 1.0)
    x[:, 5] = x[:, 5].abs() + 0.5
    x = x.to(torch.bfloat16)
    w = synth.normal(synth.stream_key(74, h), (e, h), 0.05)
    w[3, 5] = float("inf")
    w[9, 7] = float("nan")
    logits, ids, _ = lib.moe_route_topk(x.cuda(), w.cuda(), None, k)
    Lg = _np(logits)
    assert np.all(np.isposinf(Lg[:, 3])) and np.all(np.isnan(Lg[:, 9]))
    assert np.all(_np(ids)[:, 0] == 3)
    rest = [c for c in range(e) if c not in (3, 9)]
    xs, ws = _np(x).astype(np.float64), _np(w)[rest].astype(np.float64)
    L64 = xs @ ws.T
    assert np.all(np.abs(Lg[:, rest] - L64) <= 2e-6 * (np.abs(xs) @ np.abs(ws).T) + 1e-6)


def test_router_ties_pick_lower_index(lib):
    # x = 0 -> logits equal the bias; equal bias values tie
    e, h, k = 32, 256, 6
    x = torch.zeros((5, h), dtype=torch.bfloat16)
    w = synth.normal(synth.stream_key(9, 9), (e, h), 0.02)
    b = torch.zeros(e)
    b[[3, 7, 20]] = 1.0
    b[[1, 30]] = 0.5
    logits, ids, wts = lib.moe_route_topk(x.cuda(), w.cuda(), b.cuda(), k)
    assert _np(ids).tolist() == [[3, 7, 20, 1, 30, 0]] * 5
    ref = router.topk_weights(_np(logits), router.select_topk(_np(logits), k))
    assert np.allclose(_np(wts), ref, rtol=2e-6)


def test_router_k_equals_e_and_single_expert(lib):
    x, w, _ = _router_case("moe8", 9)
    logits, ids, wts = lib.moe_route_topk(x.cuda(), w.cuda(), None, 8)
    assert np.array_equal(np.sort(_np(ids), axis=1), np.tile(np.arange(8), (9, 1)))
    L = _np(logits).astype(np.float64)
    p = np.exp(L - L.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    assert np.allclose(np.take_along_axis(p, _np(ids).astype(np.int64), axis=1), _np(wts), rtol=2e-6)
    logits1, ids1, w1 = lib.moe_route_topk(x.cuda(), w[:1].contiguous().cuda(), None, 1)
    assert np.all(_np(ids1) == 0) and np.all(_np(w1) == 1.0)


# ------------------------------------------------------------------ A5 permute
@pytest.mark.parametrize("t,k,e", [(1, 1, 1), (1, 8, 256), (5, 2, 8), (64, 8, 256), (333, 3, 7),
                                   (4096, 8, 256), (100, 4, 1024), (50, 2, 4096)])
def test_permute_bit_exact(lib, t, k, e):
    rng = np.random.default_rng(t * 31 + k)
    ids = np.stack([rng.permutation(e)[:k] for _ in range(t)]).astype(np.int32)
    if t >= 64:
        ids[: t // 2, 0] = 0                 # a hot expert
    counts, offsets, perm, inv = lib.moe_permute(torch.as_tensor(ids).cuda(), e)
    rc, ro, rp, ri = permute.permute(ids, e)
    assert np.array_equal(_np(counts), rc)
    assert np.array_equal(_np(offsets), ro)
    assert np.array_equal(_np(perm), rp)
    assert np.array_equal(_np(inv), ri)


def test_permute_empty(lib):
    counts, offsets, perm, inv = lib.moe_permute(torch.zeros((0, 2), dtype=torch.int32).cuda(), 8)
    assert np.all(_np(counts) == 0) and np.all(_np(offsets) == 0) and perm.numel() == 0


# ------------------------------------------------------------------ A6 act quant
@pytest.mark.parametrize("rows,cols,f32", [(1, 128, False), (37, 2048, False), (2048, 2048, False),
                                           (19, 1024, True), (5, 7168, False)])
def test_act_quant_bit_exact(lib, rows, cols, f32):
    x = synth.normal(synth.stream_key(5, rows, cols), (rows, cols), 1.0)
    x[:, :3] *= 10
    if rows > 2:
        x[2] = 0.0                           # zero row -> s = 0, q = 0
    x = x if f32 else x.to(torch.bfloat16)
    q, s = lib.act_quant_int8(x.cuda())
    rq, rs = ffn.act_quant_int8(_np(x))
    assert np.array_equal(_np(q), rq)
    assert np.array_equal(_np(s).view(np.uint32), rs.view(np.uint32))


# ------------------------------------------------------------------ A11 INT32 core
@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("rows", [1, 16, 45])
def test_w4a8_group_accumulators_bit_exact(lib, asym, rows):
    n, k = 192, 1024
    w = _special_weights(n, k, 3)
    packed, scales, zeros = lib.quantize_int4_g128(w.cuda(), asymmetric=asym)
    dev = lib.q4_repack_device(packed, scales, zeros, n, k, asym)
    rng = np.random.default_rng(rows)
    q = rng.integers(-128, 128, size=(rows, k), dtype=np.int64).astype(np.int8)
    q[0, :128] = -128                         # extreme codes
    acc = lib.int4_w4a8_group_acc(torch.as_tensor(q).cuda(), dev, n, asym)
    qm = quant.quantize_asym(_np(w)) if asym else quant.quantize_sym(_np(w)) + (None,)
    ref = ffn.group_acc(q.astype(np.int64), ffn.widen_int8((qm[0].astype(np.int64), qm[1],
                                                            qm[2].astype(np.int64) if asym else None)))
    assert np.array_equal(_np(acc).astype(np.int64), ref)


# ------------------------------------------------------------------ linear (W4A16 core)
def test_linear_workload_parity(lib):
    x, w = synth.linear_inputs()
    packed, scales, _ = lib.quantize_int4_g128(w.cuda())
    dev = lib.q4_repack_device(packed, scales, None, 2048, 2048, False)
    y = lib.int4_linear_forward(x.cuda(), dev, 2048)
    q, s = quant.quantize_sym(_np(w))
    ref = ffn.linear_w4a16(_np(x), (q.astype(np.int64), s, None))
    assert ffn.max_rel_l2(_np(y), ref) <= 5e-3


@pytest.mark.parametrize("t,n,k,asym,dt", [(1, 64, 128, False, torch.bfloat16), (17, 192, 384, True, torch.bfloat16),
                                           (70, 128, 256, False, torch.float16), (33, 64, 1024, True, torch.float16)])
def test_linear_ragged_parity(lib, t, n, k, asym, dt):
    x = synth.normal(synth.stream_key(6, t, n), (t, k), 1.0).to(dt)
    w = _special_weights(n, k, 4) if n > 6 else synth.normal(synth.stream_key(6, 1), (n, k), 0.02)
    packed, scales, zeros = lib.quantize_int4_g128(w.cuda(), asymmetric=asym)
    dev = lib.q4_repack_device(packed, scales, zeros, n, k, asym)
    y = lib.int4_linear_forward(x.cuda(), dev, n, asym)
    from tests.helpers import oracle_qmat
    ref = ffn.linear_w4a16(_np(x), oracle_qmat(w, asym))
    assert ffn.max_rel_l2(_np(y), ref) <= 5e-3


# ------------------------------------------------------------------ generator identity
def test_generator_bit_identical_on_gpu():
    require_gpu()
    key = synth.stream_key(1, 2, 3)
    a = synth.normal(key, (1000, 777), 0.02)
    b = synth.normal(key, (1000, 777), 0.02, device="cuda").cpu()
    assert torch.equal(a, b)
    x1 = synth.tokens("moe8_w4a8", 33)
    x2 = synth.tokens("moe8_w4a8", 33, device="cuda").cpu()
    assert torch.equal(x1, x2)
