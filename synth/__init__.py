"""Seeded synthetic inputs for the INT4 g128 MoE FFN workloads.

This module is shared by the tests, the benchmark and the oracle's fitting
script.  It holds none of the method's arithmetic (no quantisation, routing,
permutation or FFN math): only counter-based random numbers and the shapes of
the workloads.

Random values come from a counter-based generator: element i of a tensor with
stream key K gets four 32-bit words h_j = mix(mix((4 i + j) xor K0) xor K1),
j = 0..3, where ``mix`` is the "lowbias32" integer hash (xorshift-multiply,
constants 0x7feb352d and 0x846ca68b, shifts 16/15/16) published by C. Wellons
(hash-prospector).  The eight 16-bit halves b_0..b_7 give
D = sum(2 b + 1) - 8 * 65536, a sum of eight centred uniforms (Irwin-Hall,
variance 2/3 per unit^2), and the sample is float32(D) * float32(sigma *
sqrt(1.5) / 131072): a unit-variance, bell-shaped value bounded by
+-4.9 sigma.  Only integer operations, one exact int->float conversion and
one correctly rounded float32 multiply are involved, so the same call gives
bit-identical tensors on the CPU and on the GPU; large weights can therefore be
made directly in device memory while the oracle regenerates any expert on the
host.
"""
import math

import numpy as np
import torch

M32 = 0xFFFFFFFF


def _mix_int(x):
    """lowbias32 on a Python int."""
    x &= M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & M32
    x ^= x >> 16
    return x


def stream_key(*parts):
    """Fold integers into a pair of 32-bit stream keys."""
    a, b = 0x2545F491, 0x9E3779B9
    for p in parts:
        p = int(p) & 0xFFFFFFFFFFFFFFFF
        a = _mix_int(a ^ (p & M32) ^ _mix_int(b))
        b = _mix_int(b + (p >> 32) + 0x632BE5AB + a)
    return a, b


def _mul32(x, c):
    """(x * c) mod 2^32 for int64 tensors x in [0, 2^32), without int64 overflow."""
    lo = x * (c & 0xFFFF)
    hi = ((x & 0xFFFF) * (c >> 16)) & 0xFFFF
    return (lo + (hi << 16)) & M32


def _mix(x):
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    return x ^ (x >> 16)


def normal_at(key, index, sigma):
    """Samples for int64 element indices ``index`` (any device, < 2^30)."""
    k0, k1 = key
    scale = torch.tensor(sigma * math.sqrt(1.5) / 131072.0, dtype=torch.float32, device=index.device)
    d = torch.zeros_like(index)
    for j in range(4):
        h = _mix(_mix(((index * 4 + j) & M32) ^ k0) ^ k1)
        d = d + ((h & 0xFFFF) * 2 + 1) + (((h >> 16) & 0xFFFF) * 2 + 1)
    d = d - 8 * 65536
    return d.to(torch.float32) * scale


def _chunked(key, index, sigma):
    chunk = 1 << 18 if index.device.type == "cpu" else 1 << 24
    out = torch.empty(index.numel(), dtype=torch.float32, device=index.device)
    for a in range(0, index.numel(), chunk):
        out[a:a + chunk] = normal_at(key, index[a:a + chunk], sigma)
    return out


def normal(key, shape, sigma, device="cpu", chunk=None):
    """A float32 tensor of the given shape, filled element by element in C order."""
    n = int(np.prod(shape))
    if chunk is None:
        chunk = 1 << 18 if torch.device(device).type == "cpu" else 1 << 24
    if n >= 1 << 30:
        raise ValueError("tensor too large for one stream")
    out = torch.empty(n, dtype=torch.float32, device=device)
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        idx = torch.arange(a, b, dtype=torch.int64, device=device)
        out[a:b] = normal_at(key, idx, sigma)
    return out.reshape(shape)


# ------------------------------------------------------------------ workloads
# Shapes of the five workloads (LLaMA-3.2-1B-shaped FFN and a 256-expert MoE).
CONFIGS = {
    "linear": dict(seed=101, t=4, n=2048, k=2048, sigma=0.02, outlier_frac=0.001,
                   outlier_mult=20.0, asymmetric=False),
    "dense": dict(seed=202, hidden=2048, inter=8192, sigma=0.02, asymmetric=True,
                  tokens=(1, 4, 16)),
    "moe8": dict(seed=303, hidden=2048, inter=1024, experts=8, top_k=2, dense_inter=8192,
                 sigma=0.02, router_sigma=0.02, asymmetric=False,
                 tokens=(1, 2, 4, 8, 16, 32, 64, 128, 256)),
    "moe8_w4a8": dict(seed=404, hidden=2048, inter=1024, experts=8, top_k=2, dense_inter=8192,
                      sigma=0.02, router_sigma=0.02, asymmetric=False, tokens=(2048,),
                      hot_channel_frac=0.01, hot_channel_mult=10.0),
    "moe256": dict(seed=505, hidden=7168, inter=2048, experts=256, top_k=8, shared=True,
                   sigma=0.02, router_sigma=0.02, asymmetric=False, zipf_s=1.1,
                   tokens=(1, 64, 4096)),
    # LoRA mode: 8 experts = low-rank adapters (rank 16) on the frozen dense 2048/8192
    # FFN that the 8-expert slice-mode layers are cut from; adapter delta ~ 20 % of the
    # base output.
    "lora8": dict(seed=606, hidden=2048, inter=8192, experts=8, top_k=2, rank=16,
                  sigma=0.02, lora_sigma_a=0.02, lora_sigma_b=0.05, router_sigma=0.02,
                  asymmetric=False, tokens=(1, 64, 2048)),
}

# Tensor tags of the stream keys.
TAG_X, TAG_W, TAG_ROUTER, TAG_GATE, TAG_UP, TAG_DOWN = 1, 2, 3, 4, 5, 6
TAG_LORA_A, TAG_LORA_B = 7, 8

# Zipf shaping of the 256-expert router: bias b_e = -zipf_s * KAPPA * ln(rank_e).
# KAPPA is fitted by synth/fit_zipf_kappa.py (see that script) so that the
# per-expert load over ranks 9..128 at T = 4096 has log-log slope -zipf_s.
ZIPF_KAPPA = 0.80


def tokens(cfg_name, t, device="cpu", salt=0):
    """bf16 tokens [t, hidden] ~ N(0, 1) (the W4A8 workload multiplies 1 % of the
    channels by 10 before the bf16 rounding)."""
    cfg = CONFIGS[cfg_name]
    h = cfg.get("hidden", cfg.get("k"))
    x = normal(stream_key(cfg["seed"], TAG_X, t, salt), (t, h), 1.0, device)
    if "hot_channel_frac" in cfg:
        ch = hot_channels(cfg_name)
        x[:, torch.as_tensor(ch, device=device)] *= cfg["hot_channel_mult"]
    return x.to(torch.bfloat16)


def hot_channels(cfg_name):
    cfg = CONFIGS[cfg_name]
    h = cfg["hidden"]
    rng = np.random.default_rng(cfg["seed"])
    return np.sort(rng.choice(h, int(h * cfg["hot_channel_frac"]), replace=False))


def linear_inputs(device="cpu"):
    """x fp16 [4, 2048] ~ N(0, 1); W fp32 [2048, 2048] ~ N(0, 0.02) with 0.1 % of the
    entries (round(0.001 N K) distinct positions) multiplied by 20."""
    cfg = CONFIGS["linear"]
    n, k = cfg["n"], cfg["k"]
    x = normal(stream_key(cfg["seed"], TAG_X), (cfg["t"], k), 1.0, device).to(torch.float16)
    w = normal(stream_key(cfg["seed"], TAG_W), (n, k), cfg["sigma"], device)
    rng = np.random.default_rng(cfg["seed"])
    pos = rng.choice(n * k, int(round(cfg["outlier_frac"] * n * k)), replace=False)
    flat = w.view(-1)
    flat[torch.as_tensor(pos, device=device)] *= cfg["outlier_mult"]
    return x, w


def dense_ffn_weights(cfg_name, device="cpu"):
    """gate [I, H], up [I, H], down [H, I] float32 of the dense FFN (dense config,
    or the dense FFN the 8-expert layers are sliced from)."""
    cfg = CONFIGS[cfg_name]
    h, i = cfg["hidden"], cfg.get("dense_inter", cfg.get("inter"))
    seed = cfg["seed"] if cfg_name == "dense" else CONFIGS["moe8"]["seed"]
    gate = normal(stream_key(seed, TAG_GATE), (i, h), cfg["sigma"], device)
    up = normal(stream_key(seed, TAG_UP), (i, h), cfg["sigma"], device)
    down = normal(stream_key(seed, TAG_DOWN), (h, i), cfg["sigma"], device)
    return gate, up, down


def slice_expert(gate, up, down, e, inter):
    """Slice mode: expert e = gate/up rows and down columns [e I, (e + 1) I) of a dense FFN."""
    sl = slice(e * inter, (e + 1) * inter)
    return gate[sl].contiguous(), up[sl].contiguous(), down[:, sl].contiguous()


def expert_weights(cfg_name, e, device="cpu"):
    """Weights of one expert: (gate [I, H], up [I, H], down [H, I]) float32.

    moe8 / moe8_w4a8: slices of the shared dense FFN (slice mode).
    moe256: expert e in [0, 256) routed, e = 256 the shared expert; each matrix
    has its own stream so any expert can be regenerated alone.
    """
    cfg = CONFIGS[cfg_name]
    h, i = cfg["hidden"], cfg["inter"]
    if cfg_name in ("moe8", "moe8_w4a8"):
        seed = CONFIGS["moe8"]["seed"]
        sig = cfg["sigma"]
        dense_i = cfg["dense_inter"]
        rows = torch.arange(e * i, (e + 1) * i, dtype=torch.int64, device=device)
        cols = torch.arange(h, dtype=torch.int64, device=device)
        idx = (rows[:, None] * h + cols[None, :]).reshape(-1)
        gate = _chunked(stream_key(seed, TAG_GATE), idx, sig).reshape(i, h)
        up = _chunked(stream_key(seed, TAG_UP), idx, sig).reshape(i, h)
        drows = torch.arange(h, dtype=torch.int64, device=device)
        dcols = torch.arange(e * i, (e + 1) * i, dtype=torch.int64, device=device)
        didx = (drows[:, None] * dense_i + dcols[None, :]).reshape(-1)
        down = _chunked(stream_key(seed, TAG_DOWN), didx, sig).reshape(h, i)
        return gate, up, down
    seed = cfg["seed"]
    gate = normal(stream_key(seed, TAG_GATE, e), (i, h), cfg["sigma"], device)
    up = normal(stream_key(seed, TAG_UP, e), (i, h), cfg["sigma"], device)
    down = normal(stream_key(seed, TAG_DOWN, e), (h, i), cfg["sigma"], device)
    return gate, up, down


def lora_base(cfg_name, device="cpu"):
    """The frozen dense FFN of a LoRA-mode layer: (gate [I, H], up [I, H], down [H, I])
    float32 -- the same dense weights the 8-expert slice-mode layers are cut from."""
    cfg = CONFIGS[cfg_name]
    seed = CONFIGS["moe8"]["seed"]
    h, i = cfg["hidden"], cfg["inter"]
    gate = normal(stream_key(seed, TAG_GATE), (i, h), cfg["sigma"], device)
    up = normal(stream_key(seed, TAG_UP), (i, h), cfg["sigma"], device)
    down = normal(stream_key(seed, TAG_DOWN), (h, i), cfg["sigma"], device)
    return gate, up, down


LORA_MATS = (("gate", "hidden", "inter"), ("up", "hidden", "inter"), ("down", "inter", "hidden"))


def lora_adapters(cfg_name, e, device="cpu", rank=None, dims=None):
    """Adapters of expert e: {"A_gate": [r, H], "B_gate": [I, r], "A_up": [r, H],
    "B_up": [I, r], "A_down": [r, I], "B_down": [H, r]} as bfloat16 tensors
    (~N(0, sigma_a) and ~N(0, sigma_b) before the bf16 rounding).  ``dims`` =
    (hidden, inter) overrides the config's sizes (small test layers)."""
    cfg = CONFIGS[cfg_name]
    r = cfg["rank"] if rank is None else rank
    h, i = (cfg["hidden"], cfg["inter"]) if dims is None else dims
    size = {"hidden": h, "inter": i}
    out = {}
    for m, (name, din, dout) in enumerate(LORA_MATS):
        a = normal(stream_key(cfg["seed"], TAG_LORA_A, m, e, r), (r, size[din]), cfg["lora_sigma_a"], device)
        b = normal(stream_key(cfg["seed"], TAG_LORA_B, m, e, r), (size[dout], r), cfg["lora_sigma_b"], device)
        out["A_" + name] = a.to(torch.bfloat16)
        out["B_" + name] = b.to(torch.bfloat16)
    return out


def router_weights(cfg_name, device="cpu", kappa=None):
    """(W_r float32 [E, H], bias float32 [E] or None).  The 256-expert layer gets the
    Zipf-shaping bias -zipf_s * kappa * ln(rank), ranks a seeded permutation of 1..E."""
    cfg = CONFIGS[cfg_name]
    seed = CONFIGS["moe8"]["seed"] if cfg_name == "moe8_w4a8" else cfg["seed"]
    w = normal(stream_key(seed, TAG_ROUTER), (cfg["experts"], cfg["hidden"]),
               cfg["router_sigma"], device)
    if "zipf_s" not in cfg:
        return w, None
    kappa = ZIPF_KAPPA if kappa is None else kappa
    rank = np.random.default_rng(seed).permutation(cfg["experts"]) + 1
    bias = (-cfg["zipf_s"] * kappa * np.log(rank.astype(np.float64))).astype(np.float32)
    return w, torch.as_tensor(bias, device=device)


def to_numpy(t):
    """CPU numpy copy of a tensor; bf16 / fp16 values widen exactly to float32."""
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.to(torch.float32)
    return t.numpy()
