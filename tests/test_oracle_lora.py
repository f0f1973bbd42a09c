"""Pins of the LoRA-mode oracle (oracle/lora.py)."""
import numpy as np
import torch

import synth
from oracle import ffn, lora, quant


def _qm(w):
    q, s = quant.quantize_sym(np.asarray(w, dtype=np.float32))
    return q.astype(np.int64), s, None


def _tiny(seed, h=128, i=128, r=2):
    rng = np.random.default_rng(seed)
    base = tuple(_qm(rng.normal(0, 0.05, shape)) for shape in ((i, h), (i, h), (h, i)))
    def ad(e):
        g = np.random.default_rng(seed * 100 + e)
        return {"A_gate": g.normal(0, 0.1, (r, h)), "B_gate": g.normal(0, 0.1, (i, r)),
                "A_up": g.normal(0, 0.1, (r, h)), "B_up": g.normal(0, 0.1, (i, r)),
                "A_down": g.normal(0, 0.1, (r, i)), "B_down": g.normal(0, 0.1, (h, r))}
    return base, ad


def test_zero_adapters_give_the_dense_ffn():
    base, _ = _tiny(1)
    zero = lambda e: {k: np.zeros_like(v) for k, v in _tiny(1)[1](e).items()}
    x = np.random.default_rng(2).normal(size=(5, 128))
    ids = np.array([[0, 3], [1, 2], [3, 0], [2, 2], [1, 0]])
    w = np.array([[0.75, 0.25], [0.5, 0.5], [0.625, 0.375], [0.25, 0.75], [1.0, 0.0]])
    out = lora.moe_lora(x, base, zero, ids, w)
    dense = ffn.swiglu_w4a16(x, *base)
    assert np.allclose(out, dense, rtol=1e-12, atol=1e-13)


def test_brute_force_definition():
    """Every output element from the definition with explicit loops over k and r."""
    h = i = 128
    r = 2
    base, ad = _tiny(3, h, i, r)
    wh = [quant.dequantize(*m) for m in base]
    x = np.random.default_rng(4).normal(size=(2, h))
    ids = np.array([[1, 0], [2, 1]])
    w = np.array([[0.6, 0.4], [0.3, 0.7]])
    out = lora.moe_lora(x, base, ad, ids, w)
    for t in range(2):
        ref = [0.0] * h
        for j in range(2):
            a = ad(int(ids[t, j]))
            hvec = []
            for c in range(i):
                g = u = 0.0
                for kk in range(h):
                    wg = wh[0][c, kk] + sum(a["B_gate"][c, q] * a["A_gate"][q, kk] for q in range(r))
                    wu = wh[1][c, kk] + sum(a["B_up"][c, q] * a["A_up"][q, kk] for q in range(r))
                    g += wg * x[t, kk]
                    u += wu * x[t, kk]
                hvec.append(g / (1.0 + np.exp(-g)) * u)
            for n in range(h):
                y = 0.0
                for c in range(i):
                    wd = wh[2][n, c] + sum(a["B_down"][n, q] * a["A_down"][q, c] for q in range(r))
                    y += wd * hvec[c]
                ref[n] += w[t, j] * y
        assert np.allclose(out[t], ref, rtol=1e-9, atol=1e-12)


def test_synthetic_adapter_scale():
    """The generated adapters move each expert's gate pre-activation by a bounded
    fraction (workload shape, checked on a slice of the layer)."""
    cfg = synth.CONFIGS["lora8"]
    gate, _, _ = synth.lora_base("lora8")
    ad = synth.lora_adapters("lora8", 3)
    x = synth.tokens("lora8", 8).to(torch.float32).numpy()
    g = x @ gate.numpy()[:256].T
    a = synth.to_numpy(ad["A_gate"]).astype(np.float64)
    b = synth.to_numpy(ad["B_gate"]).astype(np.float64)[:256]
    delta = x @ a.T @ b.T
    ratio = np.linalg.norm(delta) / np.linalg.norm(g)
    assert 0.05 < ratio < 0.6
    assert ad["A_gate"].shape == (cfg["rank"], cfg["hidden"]) and ad["B_down"].shape == (cfg["hidden"], cfg["rank"])
