"""Full-size parity of the 256-expert layer (hidden 7168, 256 experts of intermediate
2048 + one shared expert, top-8, symmetric INT4 g128, fp32 router with the Zipf bias),
built and run exactly as the benchmark runs it: bench.Workload, one step = the
library's router, then moe_int4_ffn_forward, at the benchmark's batch sizes (T = 1 and
64 decode, T = 4096 prefill) and in each arithmetic mode it reports.

The oracle routes the same tokens itself (fp64 logits) and evaluates a seeded sample of
tokens one by one; a sampled token is compared where both routings choose the same
experts (fp32 and fp64 logits may order near-ties differently; nearly all tokens
agree, which is asserted).  At the timed decode batch (T = 64) every token is compared:
the forward is given the oracle's own routing (ids and weights are inputs of
moe_int4_ffn_forward), so no token is skipped.  On the prefill kernel (T = 4096, 1280,
768) every position of four chosen experts (the most loaded, a middle one, the least
loaded one -- 11 rows at T = 4096, 1-2 rows at T = 768 / 1280 -- and the shared expert)
is checked stage by stage through moe_int4_ffn_debug, gate/up against the oracle from x
and down against the oracle on the GPU's own h.  Expert weights for the oracle come from the seeded
generator run by torch on the GPU and copied to the host (bit-identical to the host
generator, checked by test_generator_bit_identical_on_gpu), then quantised by the
oracle; nothing the library computes is fed to the oracle."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import synth
from oracle import ffn, permute as operm, quant, router
from tests.helpers import require_gpu
from tests.stagewise import check_stagewise

pytestmark = pytest.mark.gpu
CFG = "moe256"
TOL = {"w4a16": 5e-3, "w4a8": 2e-2, "w8a8": 2e-2, "mixed": 2e-2}


@pytest.fixture(scope="module")
def lib():
    require_gpu()
    import int4_group_quantized_g128_amd as lib
    return lib


def _np(t):
    return synth.to_numpy(t)


class OracleExperts:
    """Oracle-quantised experts of the layer, by (expert, bits, group); codes kept as int8."""

    def __init__(self):
        self.cache = {}

    def get(self, e, bits, group=128):
        key = (e, bits, group)
        if key not in self.cache:
            mats = synth.expert_weights(CFG, e, device="cuda")
            out = []
            for m in mats:
                w = _np(m)
                q, s = (quant.quantize_sym8(w) if bits == 8 else quant.quantize_sym2(w) if bits == 2
                        else quant.quantize_sym(w, group))
                out.append((q.astype(np.int8), s, None))
            self.cache[key] = tuple(out)
        return self.cache[key]

    def have(self, e, bits, group=128):
        return (e, bits, group) in self.cache


@pytest.fixture(scope="module")
def oracle_experts():
    return OracleExperts()


@pytest.fixture(scope="module")
def bench_mod():
    import bench
    return bench


@pytest.fixture(scope="module")
def wl4(lib, bench_mod):
    return bench_mod.Workload(lib, torch, synth, CFG, 64, "w4a16")


def _oracle_routing(x, t):
    cfg = synth.CONFIGS[CFG]
    wr, b = synth.router_weights(CFG)
    L = router.logits_fp64(x, _np(wr), _np(b))
    ids = router.select_topk(L, cfg["top_k"])
    return ids, router.topk_weights(L, ids)


def _pick(agree, ids, n, seed, bits, groups, have):
    """n agreeing tokens, preferring ones whose experts the oracle already holds."""
    cand = list(np.random.default_rng(seed).permutation(np.nonzero(agree)[0]))
    chosen = []
    while len(chosen) < n and cand:
        window = cand[:16]
        best = min(window, key=lambda r: sum(not have(int(e), bits[int(e)], groups[int(e)]) for e in ids[r]))
        chosen.append(int(best))
        cand.remove(best)
    return np.array(sorted(chosen))


def _check(lib, wl, kind, oe, nsample, seed, bits=None, groups=None):
    E = synth.CONFIGS[CFG]["experts"]
    t = wl.t
    print(f"[fullsize] {kind} T={t}: step", flush=True)
    wl.step()
    torch.cuda.synchronize()
    x = _np(synth.tokens(CFG, t))
    assert np.array_equal(_np(wl.x), x)
    ids_o, w_o = _oracle_routing(x, t)
    agree = np.all(_np(wl.ids) == ids_o, axis=1)
    assert agree.mean() >= (0.9 if t > 1 else 1.0), f"routing agrees on {agree.mean():.3f} of the tokens"
    if bits is None:
        bits = [8 if kind == "w8a8" else 4] * (E + 1)
    if groups is None:
        groups = [128] * (E + 1)
    rows = _pick(agree, ids_o, nsample, seed, bits, groups, oe.have)
    print(f"[fullsize] {kind} T={t}: oracle on tokens {rows.tolist()}", flush=True)
    expert = lambda e: oe.get(e, bits[e], groups[e])
    shared = expert(E)
    xs, ids_s, w_s = x[rows], ids_o[rows], w_o[rows]
    if kind == "w4a16":
        ref = ffn.moe_w4a16(xs, expert, ids_s, w_s, shared=shared)
    elif kind == "w4a8":
        ref = ffn.moe_w4a8(xs, expert, ids_s, w_s, shared=shared)
    elif kind == "w8a8":
        ref = ffn.moe_w8a8(xs, expert, ids_s, w_s, shared=shared)
    else:
        ref = ffn.moe_mixed(xs, expert, bits, ids_s, w_s, shared=shared, shared_bits=bits[E])
    err = ffn.max_rel_l2(_np(wl.out)[rows], ref)
    print(f"[fullsize] {kind} T={t}: max rel L2 {err:.2e}", flush=True)
    assert err <= TOL[kind]
    out = _np(wl.out)
    assert np.all(np.isfinite(out))


def test_decode_t64_w4a16(lib, wl4, oracle_experts):
    _check(lib, wl4, "w4a16", oracle_experts, 3, 1)


def test_decode_t1_w4a16(lib, wl4, oracle_experts):
    _check(lib, wl4.retoken(synth, 1), "w4a16", oracle_experts, 1, 2)


def test_prefill_t4096_w4a16(lib, wl4, oracle_experts):
    _check(lib, wl4.retoken(synth, 4096), "w4a16", oracle_experts, 2, 3)


@pytest.mark.parametrize("t", [1, 64])
def test_decode_w4a8(lib, wl4, oracle_experts, t):
    _check(lib, wl4.retoken(synth, t, "w4a8"), "w4a8", oracle_experts, 2, 4)


def test_prefill_t4096_w4a8(lib, wl4, oracle_experts):
    _check(lib, wl4.retoken(synth, 4096, "w4a8"), "w4a8", oracle_experts, 2, 5)


@pytest.mark.parametrize("t,mode", [(768, "w4a16"), (1280, "w4a8"), (512, "w4a8")])
def test_prefill_kernel_below_64_rows_per_expert(lib, wl4, oracle_experts, t, mode):
    """24, 40 and 16 routed rows per expert on average: enough work items that the
    forward takes the 128-row prefill kernel (mostly partly filled tiles)."""
    wl = wl4.retoken(synth, t, mode)
    assert lib.moe_int4_ffn_plan(wl.layer, t, wl.mode)["kernel"] == "prefill"
    _check(lib, wl, mode, oracle_experts, 2, 6 + t)


def test_decode_t64_w8a8(lib, bench_mod, oracle_experts):
    wl = bench_mod.Workload(lib, torch, synth, CFG, 64, "w8a8")
    _check(lib, wl, "w8a8", oracle_experts, 2, 6)
    del wl
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def mixed(lib, bench_mod):
    """Top 5 % of the experts by hit count (the oracle's routing of a seeded calibration
    batch) in 8 bits, the others in 4; the shared expert in 8."""
    cfg = synth.CONFIGS[CFG]
    xc = _np(synth.tokens(CFG, 4096, salt=7))
    ids_c, _ = _oracle_routing(xc, 4096)
    counts = np.bincount(ids_c.ravel(), minlength=cfg["experts"])
    bits = ffn.bits_by_hotness(counts, 0.05, shared=True)
    assert sum(b == 8 for b in bits) == 13 + 1
    wl = bench_mod.Workload(lib, torch, synth, CFG, 64, "mixed", expert_bits=bits)
    yield wl, bits
    del wl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("t", [64, 4096])
def test_mixed_widths_by_hotness(lib, mixed, oracle_experts, t):
    """INT8 activations; the decode (T = 64) and prefill (T = 4096) paths each launch one
    GEMM per width over the same tile list."""
    wl, bits = mixed
    _check(lib, wl if t == 64 else wl.retoken(synth, t), "mixed", oracle_experts, 2, 7 + t, bits=bits)


@pytest.fixture(scope="module")
def apex(lib, bench_mod):
    """APEX widths from the oracle's routing of the calibration batch: experts hit less
    than a quarter of the even share 2 bits (92 of 256), the others and the shared
    expert 4."""
    cfg = synth.CONFIGS[CFG]
    xc = _np(synth.tokens(CFG, 4096, salt=7))
    ids_c, _ = _oracle_routing(xc, 4096)
    counts = np.bincount(ids_c.ravel(), minlength=cfg["experts"])
    bits = [int(b) for b in ffn.bits_apex(counts, 0.0, 0.25, shared=True)]
    assert sum(b == 2 for b in bits) == 92 and bits[-1] == 4
    assert bits == lib.expert_bits_apex(counts.tolist(), 0.0, 0.25, shared=True)
    wl = bench_mod.Workload(lib, torch, synth, CFG, 64, "mixed", expert_bits=bits)
    yield wl, bits
    del wl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("t", [64, 4096])
def test_apex_two_bit_cold_experts(lib, apex, oracle_experts, t):
    """INT8 activations; the 2-bit experts run on the streaming kernel at both sizes."""
    wl, bits = apex
    _check(lib, wl if t == 64 else wl.retoken(synth, t), "mixed", oracle_experts, 3, 31 + t, bits=bits)


@pytest.fixture(scope="module")
def grouped(lib, bench_mod):
    """Group sizes from the oracle's routing of the calibration batch: the top 5 % of the
    experts 32, experts under a tenth of the even share 256, the others 64, shared 32."""
    cfg = synth.CONFIGS[CFG]
    xc = _np(synth.tokens(CFG, 4096, salt=7))
    ids_c, _ = _oracle_routing(xc, 4096)
    groups = ffn.groups_by_hotness(np.bincount(ids_c.ravel(), minlength=cfg["experts"]), 0.05, 0.1, shared=True)
    assert sum(g == 32 for g in groups) == 13 + 1
    wl = bench_mod.Workload(lib, torch, synth, CFG, 64, "w4a16", expert_groups=groups)
    yield wl, groups
    del wl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("t,mode", [(64, "w4a16"), (4096, "w4a8")])
def test_per_expert_groups_by_hotness(lib, grouped, oracle_experts, t, mode):
    wl, groups = grouped
    _check(lib, wl if (t, mode) == (64, "w4a16") else wl.retoken(synth, t, mode), mode, oracle_experts, 2,
           11 + t, groups=groups)


def _pool_map(fn, items):
    """The oracle's experts are independent: evaluate them on 8 threads (BLAS at 2 threads
    each); the oracle still forms every sum in its own order."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(2), ThreadPoolExecutor(8) as ex:
        return list(ex.map(fn, list(items)))


@pytest.mark.parametrize("mode", ["w4a16", "w4a8"])
def test_decode_t64_every_token(lib, wl4, oracle_experts, mode):
    """All 64 tokens of the timed decode batch against the oracle (141 routed experts +
    the shared expert), with the oracle's routing fed to the forward."""
    E = synth.CONFIGS[CFG]["experts"]
    t = 64
    x = _np(synth.tokens(CFG, t))
    ids_o, w_o = _oracle_routing(x, t)
    m = {"w4a16": lib.Q4_W4A16, "w4a8": lib.Q4_W4A8}[mode]
    assert lib.moe_int4_ffn_plan(wl4.layer, t, m)["kernel"] == "decode"
    print(f"[fullsize] every token T=64 {mode}: forward", flush=True)
    out = lib.moe_int4_ffn_forward(wl4.layer, wl4.x, torch.as_tensor(ids_o, dtype=torch.int32).cuda(),
                                   torch.as_tensor(w_o, dtype=torch.float32).cuda(), mode=m)
    torch.cuda.synchronize()
    expert = lambda e: oracle_experts.get(e, 4)
    need = sorted(set(int(e) for e in ids_o.ravel())) + [E]
    print(f"[fullsize] every token T=64 {mode}: oracle over {len(need)} experts", flush=True)
    _pool_map(expert, need)                      # quantise the needed experts (cached)
    fwd = ffn.moe_w4a16 if mode == "w4a16" else ffn.moe_w4a8
    ref = fwd(x, expert, ids_o, w_o, shared=expert(E), pmap=_pool_map)
    err = ffn.max_rel_l2(_np(out), ref)
    print(f"[fullsize] every token T=64 {mode}: max rel L2 {err:.2e}", flush=True)
    assert err <= TOL[mode]


@pytest.mark.parametrize("t,mode", [(4096, "w4a16"), (4096, "w4a8"), (768, "w4a16"), (1280, "w4a8")])
def test_prefill_chosen_experts_every_position(lib, wl4, oracle_experts, t, mode):
    """Every position of the most loaded expert, a middle one, the least loaded one and
    the shared expert, stage by stage, on the prefill kernel.  At T = 4096 the least
    loaded expert has 11 rows (one partly filled 128-row tile); at T = 768 / 1280 it has
    1 / 2 rows."""
    cfg = synth.CONFIGS[CFG]
    E = cfg["experts"]
    x = synth.tokens(CFG, t)
    ids_o, w_o = _oracle_routing(_np(x), t)
    counts = np.bincount(ids_o.ravel(), minlength=E)
    order = np.argsort(-counts, kind="stable")
    nz = order[counts[order] > 0]
    chosen = [int(nz[0]), int(nz[len(nz) // 2]), int(nz[-1]), E]
    rows = [int(counts[e]) if e < E else t for e in chosen]
    print(f"[fullsize] T={t} {mode}: experts {chosen} with rows {rows}", flush=True)
    assert rows[2] <= (16 if t >= 4096 else 8)
    m = {"w4a16": lib.Q4_W4A16, "w4a8": lib.Q4_W4A8}[mode]
    assert lib.moe_int4_ffn_plan(wl4.layer, t, m)["kernel"] == "prefill"
    _pool_map(lambda e: oracle_experts.get(e, 4), chosen)
    check_stagewise(lib, wl4.layer, lambda e: oracle_experts.get(e, 4), x, ids_o, w_o, m, shared=True,
                    experts=chosen, gate_up_rows=32)
