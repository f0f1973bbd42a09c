"""Shared test helpers: building oracle experts and device layers from the seeded
synthetic weights.  The oracle side only ever sees generator output (CPU tensors);
nothing computed by the HIP library is fed back into the oracle."""
import numpy as np
import pytest
import torch

import synth
from oracle import quant


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def oracle_qmat(w, asym):
    """fp32 weight (tensor or array) -> oracle (q int64, s f16, z int64 | None)."""
    w = synth.to_numpy(w) if isinstance(w, torch.Tensor) else np.asarray(w, dtype=np.float32)
    if asym:
        q, s, z = quant.quantize_asym(w)
        return q.astype(np.int64), s, z.astype(np.int64)
    q, s = quant.quantize_sym(w)
    return q.astype(np.int64), s, None


class OracleExperts:
    """Lazily generated + oracle-quantised experts (CPU), cached by index."""

    def __init__(self, make, asym):
        self.make = make        # e -> (gate, up, down) fp32 CPU tensors
        self.asym = asym
        self.cache = {}

    def __call__(self, e):
        if e not in self.cache:
            g, u, d = self.make(e)
            self.cache[e] = (oracle_qmat(g, self.asym), oracle_qmat(u, self.asym), oracle_qmat(d, self.asym))
        return self.cache[e]


def build_gpu_layer(lib, make, num_experts, hidden, inter, top_k, asym=False, shared=False, device="cuda"):
    """Device layer from the same generator, quantised by the library's kernels."""
    layer = lib.MoELayer(num_experts, hidden, inter, top_k, asymmetric=asym, shared=shared, device=device)
    for e in range(num_experts + (1 if shared else 0)):
        g, u, d = make(e, device)
        layer.set_expert(e, g, u, d)
    torch.cuda.synchronize()
    return layer


def random_expert_maker(seed, hidden, inter, sigma=0.05):
    def make(e, device="cpu"):
        return (synth.normal(synth.stream_key(seed, 1, e), (inter, hidden), sigma, device),
                synth.normal(synth.stream_key(seed, 2, e), (inter, hidden), sigma, device),
                synth.normal(synth.stream_key(seed, 3, e), (hidden, inter), sigma, device))
    return make


def rel_l2_rows(y, ref):
    from oracle.ffn import max_rel_l2
    return max_rel_l2(y, ref)


def y_positions(v):
    """Per-position routed outputs from the debug views: the fp32 sum of the down
    projection's K slices in slice order (the forward's own combine order); whole rows
    when the forward does not split K.  Returned as float64."""
    y = synth.to_numpy(v["y"]).astype(np.float32)
    acc = y[0].copy()
    for s in range(1, y.shape[0]):
        acc = acc + y[s]
    return acc.astype(np.float64)


def k_slice(qm, g0, g1):
    """Columns [128 g0, 128 g1) of an oracle quantised matrix (q, s, z) (groups of 128)."""
    q, s, z = qm
    return (q[:, 128 * g0:128 * g1], s[:, g0:g1], None if z is None else z[:, g0:g1])
