"""LoRA-mode experts (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Page "高效大语言模型推理实践：INT4量化与MoE架构的融合探索", 第三阶段 (and its English
summary, item 3 of the approach): in LoRA mode every expert starts from the frozen
dense FFN weights plus its own LoRA adapters.  Here the frozen dense weights are the
INT4 g128 matrices (their dequantised values W_hat), and expert e of matrix m in
{gate, up, down} is

    W_m,e = W_hat_m + B_m,e A_m,e,      A_m,e [r, in], B_m,e [out, r],

with the adapters given as real numbers (bf16 values; any LoRA scaling is taken to be
folded into B).  The expert is the SwiGLU FFN of those matrices,

    FFN_e(x) = W_down,e (silu(W_gate,e x) * (W_up,e x)),

and the layer output is out[t] = sum_j w[t, j] FFN_{ids[t, j]}(x[t]) (MoE section of
page "大模型之Dense、MoE与量化").  Everything is evaluated in float64 from the merged
matrices, exactly as defined.

Pinned by (tests/test_oracle_lora.py): zero adapters reduce every expert to the dense
INT4 FFN (so any routing with weights summing to 1 gives the dense output); brute-force
element-by-element evaluation of the definition with Python loops on tiny shapes.
"""
import numpy as np

from .ffn import silu
from .quant import dequantize


def merged(qm, a, b):
    """W_hat + B A in float64 for a quantised base (q, s, z) and adapters A, B."""
    w = dequantize(*qm)
    return w + np.asarray(b, dtype=np.float64) @ np.asarray(a, dtype=np.float64)


def lora_expert(x, base, ad):
    """FFN_e(x) for base = (gate, up, down) quantised matrices and ad = the expert's
    adapters {"A_gate", "B_gate", "A_up", "B_up", "A_down", "B_down"}."""
    x64 = np.asarray(x, dtype=np.float64)
    wg = merged(base[0], ad["A_gate"], ad["B_gate"])
    wu = merged(base[1], ad["A_up"], ad["B_up"])
    wd = merged(base[2], ad["A_down"], ad["B_down"])
    return (silu(x64 @ wg.T) * (x64 @ wu.T)) @ wd.T


def moe_lora(x, base, adapters, ids, weights):
    """``adapters(e)`` returns the adapters of expert e (arrays)."""
    x64 = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids)
    w = np.asarray(weights, dtype=np.float64)
    out = np.zeros((x64.shape[0], x64.shape[1]), dtype=np.float64)
    for e in np.unique(ids):
        rows, cols = np.nonzero(ids == e)
        y = lora_expert(x64[rows], base, adapters(int(e)))
        for i, (r, c) in enumerate(zip(rows, cols)):
            out[r] += w[r, c] * y[i]
    return out
