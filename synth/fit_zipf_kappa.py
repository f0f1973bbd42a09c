"""Fit the Zipf-shaping constant of the 256-expert router bias (workload shaping).

Run as ``python -m synth.fit_zipf_kappa``; the result is stored as
``synth.ZIPF_KAPPA`` and checked by ``tests/test_synth_zipf.py``.

The 256-expert workload asks for an expert load that follows Zipf(s = 1.1).  An
exact Zipf load is infeasible with top-8 routing (the first expert would need more
than every token), so the router bias is b_e = -s * kappa * ln(r_e) with r_e a
seeded rank permutation, and kappa is chosen so that the realised per-expert load,
sorted descending, has a log-log slope of -s over ranks 9..128 at T = 4096.

This is a property of the synthetic inputs, not of the method: the routing that
realises the load is passed in (the script uses the CPU oracle's fp64 logits and
top-k rule, as a script that writes stored values for the tests may).  Nothing in
this module computes a step of the method itself.
"""
import numpy as np

import synth

RANKS = (9, 128)   # the ranks whose load the slope is fitted over


def slope_of_load(load, ranks=RANKS):
    """Log-log slope of the per-expert load, sorted descending, over ``ranks`` (a zero
    load counts as 0.5)."""
    srt = np.sort(np.asarray(load, dtype=np.float64))[::-1]
    r = np.arange(ranks[0], ranks[1] + 1)
    return float(np.polyfit(np.log(r), np.log(np.maximum(srt[r - 1], 0.5)), 1)[0])


def load_slope(ids, num_experts, ranks=RANKS):
    """(slope_of_load of the routed ids' per-expert load, the load sorted descending)."""
    load = np.sort(np.bincount(np.asarray(ids).ravel(), minlength=num_experts))[::-1].astype(np.float64)
    return slope_of_load(load, ranks), load


def kl_to_zipf(load, s):
    """KL(realised load share || Zipf(s) over the same ranks), in nats; the realised
    shares are the descending per-expert loads normalised to sum 1."""
    load = np.sort(np.asarray(load, dtype=np.float64))[::-1]
    p = load / load.sum()
    q = np.arange(1, len(p) + 1, dtype=np.float64) ** (-s)
    q /= q.sum()
    nz = p > 0
    return float(np.sum(p[nz] * np.log(p[nz] / q[nz])))


def fit(route, t=4096, iters=14):
    """Bisection on kappa; ``route(kappa) -> ids [t][k]`` routes the seeded batch."""
    cfg = synth.CONFIGS["moe256"]
    lo, hi = 0.2, 2.0
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        sl, _ = load_slope(route(mid), cfg["experts"])
        if sl > -cfg["zipf_s"]:
            lo = mid
        else:
            hi = mid
    return round(0.5 * (lo + hi), 3)


def main():
    from oracle import router   # the stored constant comes from the oracle's routing

    cfg = synth.CONFIGS["moe256"]
    t = 4096
    x = synth.to_numpy(synth.tokens("moe256", t))
    w, bias1 = synth.router_weights("moe256", kappa=1.0)
    base = router.logits_fp64(x, synth.to_numpy(w), None)
    unit = synth.to_numpy(bias1).astype(np.float64)        # -s * ln(rank) with kappa = 1

    def route(kappa):
        return router.select_topk(base + kappa * unit[None, :], cfg["top_k"])

    kappa = fit(route, t)
    sl, load = load_slope(route(kappa), cfg["experts"])
    print(f"kappa={kappa} slope={sl:.3f} top={load[0] / t:.3f} of tokens, "
          f"min={load[-1]:.0f}, touched={np.count_nonzero(load)}, KL to Zipf={kl_to_zipf(load, cfg['zipf_s']):.4f}")


if __name__ == "__main__":
    main()
