"""Router: logits, top-k selection and renormalised combine weights (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Page "大模型之Dense、MoE与量化", MoE section: the router is a Linear layer that
scores the experts, a few experts are picked, and their outputs are combined in
proportion to the scores.  Page "MoE推理优化实战：4bit存储+INT8计算的W4A8路线解析",
§3.2: the router is kept in floating point, not INT8 (this build keeps it in
float32).

Readings (listed in the design doc):

* logits L = x W_r^T (+ b), the bias also taking part in the selection;
* selection on the float32 logits: order by (-L[e], e), i.e. descending logit,
  equal logits -> lower expert index, first k kept;
* weights w_j = exp(L_j - L_max) / sum_{i in selected} exp(L_i - L_max), which
  is the softmax over all E followed by renormalising the selected k.

Pinned by (tests/test_oracle_router.py): sum of weights = 1; k = E reproduces
the full softmax (computed independently with scipy.special.softmax); E = 1
gives weight exactly 1.0; constructed exact ties pick the lower index; the
selected set equals a brute-force lexsort and the k largest values.
"""
import numpy as np


def logits_fp64(x, w_router, bias=None):
    """fp64 logits [T, E] from x [T, H] (bf16 values widened) and W_r [E, H]."""
    x64 = np.asarray(x, dtype=np.float64)
    w64 = np.asarray(w_router, dtype=np.float64)
    out = x64 @ w64.T
    if bias is not None:
        out = out + np.asarray(bias, dtype=np.float64)[None, :]
    return out


def select_topk(logits, k):
    """Top-k expert ids per row of a logit array: descending value, ties -> lower index."""
    L = np.asarray(logits)
    t, e = L.shape
    if not 1 <= k <= e:
        raise ValueError("need 1 <= k <= E")
    ids = np.empty((t, k), dtype=np.int32)
    for r in range(t):
        # python's sort is stable; the key makes the order explicit anyway
        order = sorted(range(e), key=lambda j: (-float(L[r, j]), j))
        ids[r] = order[:k]
    return ids


def topk_weights(logits, ids):
    """Renormalised softmax weights of the selected experts (fp64)."""
    L = np.asarray(logits, dtype=np.float64)
    t, k = ids.shape
    w = np.empty((t, k), dtype=np.float64)
    for r in range(t):
        sel = L[r, ids[r]]
        m = np.max(L[r])
        ex = np.exp(sel - m)
        w[r] = ex / np.sum(ex)
    return w


def route(x, w_router, bias, k):
    """Reference routing from fp64 logits: (logits64, ids, weights64)."""
    L = logits_fp64(x, w_router, bias)
    ids = select_topk(L, k)
    return L, ids, topk_weights(L, ids)
