"""The 256-expert workload's Zipf-shaped load (workload shaping, not the method).

Routes the seeded T = 4096 batch with the oracle (fp64 logits plus the stored bias at
synth.ZIPF_KAPPA, the oracle's top-k rule) and checks that the realised per-expert
load, sorted descending, falls with a log-log slope of -1.1 +- 0.05 over ranks
9..128, the stated reading of "Zipf(s = 1.1) expert load" under top-8 routing.
"""
import numpy as np
import pytest

import synth
from oracle import router
from synth import fit_zipf_kappa as fz


@pytest.fixture(scope="module")
def routed_4096():
    cfg = synth.CONFIGS["moe256"]
    x = synth.to_numpy(synth.tokens("moe256", 4096))
    w, b = synth.router_weights("moe256")
    L = router.logits_fp64(x, synth.to_numpy(w), synth.to_numpy(b))
    return router.select_topk(L, cfg["top_k"])


def test_stored_kappa_gives_zipf_slope(routed_4096):
    cfg = synth.CONFIGS["moe256"]
    assert synth.ZIPF_KAPPA == 0.80
    slope, load = fz.load_slope(routed_4096, cfg["experts"])
    assert abs(slope - (-cfg["zipf_s"])) <= 0.05, slope
    # every token lands on top_k distinct experts
    assert load.sum() == 4096 * cfg["top_k"]
    # the head is heavy (the top expert takes most tokens) and the tail is not empty
    assert load[0] > 0.4 * 4096
    assert np.count_nonzero(load) == cfg["experts"]


def test_unbiased_router_is_not_zipf(routed_4096):
    """Without the bias (kappa = 0) the load is far flatter: the bias is what shapes it."""
    cfg = synth.CONFIGS["moe256"]
    x = synth.to_numpy(synth.tokens("moe256", 1024))
    w, _ = synth.router_weights("moe256")
    ids = router.select_topk(router.logits_fp64(x, synth.to_numpy(w), None), cfg["top_k"])
    slope, _ = fz.load_slope(ids, cfg["experts"])
    assert slope > -0.6, slope


def test_kl_to_zipf():
    s = 1.1
    q = np.arange(1, 257, dtype=np.float64) ** (-s)
    assert fz.kl_to_zipf(q * 1000.0, s) == pytest.approx(0.0, abs=1e-12)
    # a uniform load over 256 experts: KL = sum (1/256) ln((1/256) / q_r)
    qn = q / q.sum()
    expect = float(np.sum((1 / 256) * np.log((1 / 256) / qn)))
    assert fz.kl_to_zipf(np.ones(256), s) == pytest.approx(expect, rel=1e-12)
    # order of the input does not matter (the load is sorted first)
    rng = np.random.default_rng(0)
    load = rng.integers(0, 50, 256)
    assert fz.kl_to_zipf(load, s) == pytest.approx(fz.kl_to_zipf(rng.permutation(load), s), rel=1e-12)
