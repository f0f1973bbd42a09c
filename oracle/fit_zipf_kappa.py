"""Fit the Zipf-shaping constant of the 256-expert router bias (workload shaping).

TEST INFRASTRUCTURE ONLY.  Run as ``python -m oracle.fit_zipf_kappa``.

The 256-expert workload asks for an expert load that follows Zipf(s = 1.1).
An exact Zipf load is infeasible with top-8 routing (the first expert would
need more than every token), so the router bias is b_e = -s * kappa * ln(r_e)
with r_e a seeded rank permutation, and kappa is chosen so that the realised
per-expert load, sorted descending, has a log-log slope of -s over ranks
9..128 at T = 4096.  Routing uses the oracle's fp64 logits and its top-k rule.
The fitted value is stored as synth.ZIPF_KAPPA.  Parity unpinned: this is a
property of the synthetic workload, not of the method.
"""
import numpy as np

import synth
from oracle import router


def slope_for(base_logits, rank_bias_unit, kappa, k, s):
    L = base_logits + kappa * rank_bias_unit[None, :]
    ids = router.select_topk(L, k)
    load = np.sort(np.bincount(ids.ravel(), minlength=L.shape[1]))[::-1].astype(np.float64)
    r = np.arange(9, 129)
    y = np.log(np.maximum(load[r - 1], 0.5))
    return np.polyfit(np.log(r), y, 1)[0], load


def main():
    cfg = synth.CONFIGS["moe256"]
    t = 4096
    x = synth.to_numpy(synth.tokens("moe256", t))
    w, bias1 = synth.router_weights("moe256", kappa=1.0)
    base = router.logits_fp64(x, synth.to_numpy(w), None)
    unit = synth.to_numpy(bias1).astype(np.float64)        # -s * ln(rank) with kappa = 1
    lo, hi = 0.2, 2.0
    for _ in range(14):
        mid = 0.5 * (lo + hi)
        sl, _ = slope_for(base, unit, mid, cfg["top_k"], cfg["zipf_s"])
        if sl > -cfg["zipf_s"]:
            lo = mid
        else:
            hi = mid
    kappa = round(0.5 * (lo + hi), 3)
    sl, load = slope_for(base, unit, kappa, cfg["top_k"], cfg["zipf_s"])
    print(f"kappa={kappa} slope={sl:.3f} top={load[0] / t:.3f} of tokens, "
          f"min={load[-1]:.0f}, touched={np.count_nonzero(load)}")


if __name__ == "__main__":
    main()
