"""Benchmark of the INT4 g128 MoE SwiGLU FFN forward on one MI355X.

A step is one pass of the hot path over one batch: fp32 router (logits, softmax,
top-k) -> permutation -> fused gate/up + SwiGLU grouped GEMM -> down grouped GEMM ->
weighted combine (+ the shared expert), all through the C ABI of libq4moe.so.

Default workload: the large MoE layer on one GPU (hidden 7168, 256 routed experts of
intermediate 2048 plus one shared expert, top-8, fp32 router with a Zipf-shaping
bias, symmetric INT4 g128 weights, 5.84 GB packed), decode batch T = 64, W4A16.
Weights and tokens are seeded synthetic data made on the GPU by the counter-based
generator in ``synth`` (the oracle can regenerate any expert on the host).

Prints one JSON line (see the keys below).  ``--gpus N`` with N > 1 exits: this
build runs on one GPU.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
# HBM counter summaries (rocprofv3 FETCH_SIZE / WRITE_SIZE, copy-calibrated) of the gate/up kernel
# by (layer, tokens, mode) of the main line; used as roofline traffic only while the GEMM sources
# still hash the same
TRAFFIC_PROFILES = {
    ("moe256", 64, "w4a16"): os.path.join(ROOT, "profiles", "k_gemm_gate_up_moe256_T64_w4a16.txt"),
    ("moe256", 1, "w4a16"): os.path.join(ROOT, "profiles", "k_gemm_decode_moe256_T1_w4a16.txt"),
    ("moe256", 4096, "w4a16"): os.path.join(ROOT, "profiles", "k_gemm_pf_moe256_T4096_w4a16.txt"),
    ("moe256", 4096, "w4a8"): os.path.join(ROOT, "profiles", "k_gemm_pf_moe256_T4096_w4a8.txt"),
    ("moe8_w4a8", 2048, "w4a8"): os.path.join(ROOT, "profiles", "k_gemm_pf_moe8_T2048_w4a8.txt"),
}
WARM_SECONDS = 0.3             # minimum untimed graph replay time before a timed region
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
INT8_PEAK_TOPS = 5000.0        # dense int8 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", choices=["moe256", "moe8_w4a8"], default="moe256",
                   help="layer of the main line: the 256-expert layer, or the 8-expert W4A8 prefill layer")
    p.add_argument("--tokens", type=int, default=64)
    p.add_argument("--mode", choices=["w4a16", "w4a8", "w8a8"], default="w4a16")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-tokens", type=int, default=2, help="tokens in the oracle's timed sample")
    p.add_argument("--no-extra", action="store_true", help="skip the secondary workloads")
    p.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replays")
    p.add_argument("--no-cold", action="store_true",
                   help="skip the cache-flushed timing of the main line (profiler runs: the kernel "
                        "trace averages then hold warm steps only, as the live averages do)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 512 MiB device copy (HBM counter calibration)")
    return p.parse_args()


class Workload:
    """Device-resident layer + router + tokens + preallocated buffers for one config."""

    def __init__(self, lib, torch, synth, cfg_name, t, mode, expert_bits=None, expert_groups=None):
        """mode "w4a16" / "w4a8" / "w8a8", or "mixed": per-expert widths ``expert_bits``
        (4 or 8 per expert and the shared expert) with INT8 activations; ``expert_groups``:
        per-expert group sizes of the INT4 weights (modes w4a16 / w4a8)."""
        self.lib, self.torch = lib, torch
        cfg = synth.CONFIGS[cfg_name]
        self.cfg_name, self.cfg, self.t = cfg_name, cfg, t
        self.mode = {"w4a16": lib.Q4_W4A16, "w4a8": lib.Q4_W4A8, "w8a8": lib.Q4_W8A8, "mixed": lib.Q4_W4A8}[mode]
        self.wbits = 8 if mode == "w8a8" else 4
        e, h, i, k = cfg["experts"], cfg["hidden"], cfg["inter"], cfg["top_k"]
        shared = bool(cfg.get("shared", False))
        self.layer = lib.MoELayer(e, h, i, k, asymmetric=cfg["asymmetric"], shared=shared, weight_bits=self.wbits,
                                  expert_bits=expert_bits if mode == "mixed" else None,
                                  expert_groups=expert_groups)
        for j in range(e + (1 if shared else 0)):
            g, u, d = synth.expert_weights(cfg_name, j, device="cuda")
            self.layer.set_expert(j, g, u, d)
            del g, u, d
        self.wr, self.bias = synth.router_weights(cfg_name, device="cuda")
        self.x = synth.tokens(cfg_name, t, device="cuda")
        dev = "cuda"
        self.logits = torch.empty((t, e), dtype=torch.float32, device=dev)
        self.ids = torch.empty((t, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((t, k), dtype=torch.float32, device=dev)
        self.rws_bytes = int(lib._lib.raw.moe_route_workspace_bytes(t, h, e))
        self.rws = torch.empty(max(self.rws_bytes, 1), dtype=torch.uint8, device=dev)
        self.out = torch.empty((t, h), dtype=torch.bfloat16, device=dev)
        self.ws_bytes = self.layer.workspace_bytes(t, self.mode)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    def retoken(self, synth, t, mode=None):
        """Same layer and router, a new batch of t tokens with its own buffers (and
        optionally the other arithmetic mode)."""
        torch = self.torch
        other = Workload.__new__(Workload)
        other.__dict__.update(self.__dict__)
        other.t = t
        if mode is not None:
            other.mode = self.lib.Q4_W4A8 if mode == "w4a8" else self.lib.Q4_W4A16
        e, h, k = self.cfg["experts"], self.cfg["hidden"], self.cfg["top_k"]
        other.x = synth.tokens(self.cfg_name, t, device="cuda")
        other.logits = torch.empty((t, e), dtype=torch.float32, device="cuda")
        other.ids = torch.empty((t, k), dtype=torch.int32, device="cuda")
        other.w = torch.empty((t, k), dtype=torch.float32, device="cuda")
        other.rws_bytes = int(self.lib._lib.raw.moe_route_workspace_bytes(t, h, e))
        other.rws = torch.empty(max(other.rws_bytes, 1), dtype=torch.uint8, device="cuda")
        other.out = torch.empty((t, h), dtype=torch.bfloat16, device="cuda")
        other.ws_bytes = self.layer.workspace_bytes(t, other.mode)
        other.ws = torch.empty(max(other.ws_bytes, 1), dtype=torch.uint8, device="cuda")
        return other

    def step(self):
        L = self.lib._lib
        raw, P, st = L.raw, L._ptr, L._stream()
        e, h, k = self.cfg["experts"], self.cfg["hidden"], self.cfg["top_k"]
        rc = raw.moe_route_topk(P(self.x), P(self.wr), P(self.bias), self.t, h, e, k, P(self.logits),
                                P(self.ids), P(self.w), P(self.rws), self.rws_bytes, st)
        if rc:
            raise L.Q4Error("moe_route_topk", rc)
        rc = raw.moe_int4_ffn_forward(L.ctypes.byref(self.layer.desc), P(self.x), self.t, P(self.ids), P(self.w),
                                      self.mode, P(self.out), P(self.ws), self.ws_bytes, st)
        if rc:
            raise L.Q4Error("moe_int4_ffn_forward", rc)

    def touched_experts(self):
        """Experts with at least one routed row (+ the shared expert)."""
        ids = [int(v) for v in self.torch.unique(self.ids.cpu()).tolist()]
        return ids + ([self.cfg["experts"]] if self.layer.shared else [])

    def touched(self):
        return len(self.touched_experts())

    def expert_bytes(self, bits=None, group=128):
        """Canonical packed bytes of one expert: codes (4- or 8-bit) + fp16 scales (+ zero points)."""
        h, i = self.cfg["hidden"], self.cfg["inter"]
        b = bits or self.wbits             # code bits per weight
        gu = 2 * i * h * b // 8 + 2 * i * (h // group) * 2
        dn = h * i * b // 8 + h * (i // group) * 2
        if self.cfg["asymmetric"]:
            gu += 2 * i * ((h // 128 + 1) // 2)
            dn += h * ((i // 128 + 1) // 2)
        return gu, dn

    def touched_bytes(self):
        """Canonical bytes (gate/up, down) of the touched experts, each at its own width."""
        gu = dn = 0
        for e in self.touched_experts():
            a, b = self.expert_bytes(self.layer.bits[e], self.layer.groups[e])
            gu, dn = gu + a, dn + b
        return gu, dn

    def flops(self):
        """Algorithmic matrix flops of the expert GEMMs (routed slots + shared rows)."""
        h, i, k = self.cfg["hidden"], self.cfg["inter"], self.cfg["top_k"]
        rows = self.t * (k + (1 if self.layer.shared else 0))
        return 2.0 * rows * 3 * h * i


class LoraWorkload:
    """LoRA-mode layer (frozen INT4 dense FFN + rank-r adapters per expert) + router +
    tokens + preallocated buffers; a step is router -> moe_lora_ffn_forward."""

    def __init__(self, lib, torch, synth, cfg_name, t):
        self.lib, self.torch = lib, torch
        cfg = synth.CONFIGS[cfg_name]
        self.cfg_name, self.cfg, self.t = cfg_name, cfg, t
        self.mode = None
        e, h, i, k, r = cfg["experts"], cfg["hidden"], cfg["inter"], cfg["top_k"], cfg["rank"]
        self.layer = lib.LoRALayer(e, h, i, k, r)
        self.layer.set_base(*(m.cuda() for m in synth.lora_base(cfg_name)))
        for j in range(e):
            self.layer.set_adapters(j, {n: v.cuda() for n, v in synth.lora_adapters(cfg_name, j).items()})
        self.wr, _ = synth.router_weights(cfg_name, device="cuda")
        self.x = synth.tokens(cfg_name, t, device="cuda")
        self.logits = torch.empty((t, e), dtype=torch.float32, device="cuda")
        self.ids = torch.empty((t, k), dtype=torch.int32, device="cuda")
        self.w = torch.empty((t, k), dtype=torch.float32, device="cuda")
        self.rws_bytes = int(lib._lib.raw.moe_route_workspace_bytes(t, h, e))
        self.rws = torch.empty(max(self.rws_bytes, 1), dtype=torch.uint8, device="cuda")
        self.out = torch.empty((t, h), dtype=torch.bfloat16, device="cuda")
        self.ws_bytes = self.layer.workspace_bytes(t)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()

    def step(self):
        L = self.lib._lib
        raw, P, st = L.raw, L._ptr, L._stream()
        e, h, k = self.cfg["experts"], self.cfg["hidden"], self.cfg["top_k"]
        rc = raw.moe_route_topk(P(self.x), P(self.wr), None, self.t, h, e, k, P(self.logits), P(self.ids),
                                P(self.w), P(self.rws), self.rws_bytes, st)
        if rc:
            raise L.Q4Error("moe_route_topk", rc)
        rc = raw.moe_lora_ffn_forward(L.ctypes.byref(self.layer.desc), P(self.x), self.t, P(self.ids), P(self.w),
                                      P(self.out), P(self.ws), self.ws_bytes, st)
        if rc:
            raise L.Q4Error("moe_lora_ffn_forward", rc)

    def summary(self, sec, cold_sec=None):
        h, i, r, k = self.cfg["hidden"], self.cfg["inter"], self.cfg["rank"], self.cfg["top_k"]
        flops = 2.0 * self.t * 3 * h * i + 2.0 * self.t * k * 3 * r * (h + i)
        res = {"tokens": self.t, "tokens_per_s": self.t / sec, "ms_per_step": sec * 1e3,
               "weight_bytes": self.layer.weight_bytes(),
               "effective_weight_GBps": self.layer.weight_bytes() / sec / 1e9,
               "hbm_frac": self.layer.weight_bytes() / sec / 1e9 / HBM_PEAK_GBS,
               "mfma_frac": flops / sec / 1e12 / BF16_PEAK_TFLOPS}
        if cold_sec is not None:
            res["ms_per_step_cold"] = cold_sec * 1e3
            res["hbm_frac_cold"] = self.layer.weight_bytes() / cold_sec / 1e9 / HBM_PEAK_GBS
        return res


class DenseWorkload(Workload):
    """The LLaMA-3.2-1B-shaped dense SwiGLU FFN (hidden 2048, intermediate 8192,
    asymmetric INT4 g128) as a one-expert layer with weight 1 and no router; a step is
    moe_int4_ffn_forward alone."""

    def __init__(self, lib, torch, synth, t, mode):
        self.lib, self.torch = lib, torch
        base = synth.CONFIGS["dense"]
        self.cfg_name, self.cfg, self.t = "dense", dict(base, experts=1, top_k=1), t
        self.mode = {"w4a16": lib.Q4_W4A16, "w4a8": lib.Q4_W4A8}[mode]
        self.wbits = 4
        h, i = base["hidden"], base["inter"]
        self.layer = lib.MoELayer(1, h, i, 1, asymmetric=True)
        g, u, d = synth.dense_ffn_weights("dense", device="cuda")
        self.layer.set_expert(0, g, u, d)
        del g, u, d
        self.x = synth.tokens("dense", t, device="cuda")
        self.ids = torch.zeros((t, 1), dtype=torch.int32, device="cuda")
        self.w = torch.ones((t, 1), dtype=torch.float32, device="cuda")
        self.out = torch.empty((t, h), dtype=torch.bfloat16, device="cuda")
        self.ws_bytes = self.layer.workspace_bytes(t, self.mode)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()

    def step(self):
        L = self.lib._lib
        raw, P, st = L.raw, L._ptr, L._stream()
        rc = raw.moe_int4_ffn_forward(L.ctypes.byref(self.layer.desc), P(self.x), self.t, P(self.ids), P(self.w),
                                      self.mode, P(self.out), P(self.ws), self.ws_bytes, st)
        if rc:
            raise L.Q4Error("moe_int4_ffn_forward", rc)


class LinearWorkload:
    """The single INT4 g128 linear y = x W^T (x fp16 [4, 2048], W [2048, 2048] with 0.1 %
    outliers x20, symmetric), quantised and repacked on the GPU; a step is
    int4_linear_forward (fp32 output)."""

    def __init__(self, lib, torch, synth):
        self.lib, self.torch = lib, torch
        cfg = synth.CONFIGS["linear"]
        self.cfg, self.t, self.mode = cfg, cfg["t"], None
        self.n, self.k = cfg["n"], cfg["k"]
        self.x, w = synth.linear_inputs(device="cuda")
        packed, scales, zeros = lib.quantize_int4_g128(w)
        self.w_dev = lib.q4_repack_device(packed, scales, zeros, self.n, self.k)
        del w, packed, scales, zeros
        self.y = torch.empty((self.t, self.n), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()

    def step(self):
        L = self.lib._lib
        rc = L.raw.int4_linear_forward(L._ptr(self.x), L.Q4_F16, self.t, self.k, L._ptr(self.w_dev), self.n, 0,
                                       L._ptr(self.y), L._stream())
        if rc:
            raise L.Q4Error("int4_linear_forward", rc)

    def summary(self, sec, cold_sec=None):
        g = self.k // 128
        wbytes = self.n * self.k // 2 + 2 * self.n * g       # nibbles + fp16 scales
        res = {"tokens": self.t, "tokens_per_s": self.t / sec, "ms_per_step": sec * 1e3, "weight_bytes": wbytes,
               "effective_weight_GBps": wbytes / sec / 1e9, "hbm_frac": wbytes / sec / 1e9 / HBM_PEAK_GBS,
               "flops": 2.0 * self.t * self.n * self.k}
        if cold_sec is not None:
            res["ms_per_step_cold"] = cold_sec * 1e3
            res["hbm_frac_cold"] = wbytes / cold_sec / 1e9 / HBM_PEAK_GBS
        return res


def expert_load(wl):
    """Realised per-expert load of the batch (routed slots per expert, from the router's
    ids): the sorted histogram's head, how many experts are touched, the smallest
    non-zero load and, for the Zipf-shaped router, the log-log slope over ranks 9..128
    and the KL divergence of the load shares from Zipf(s)."""
    import numpy as np
    from synth import fit_zipf_kappa as fz
    E = wl.cfg["experts"]
    if E <= 1:
        return None
    counts = np.bincount(wl.ids.cpu().numpy().ravel(), minlength=E)
    srt = np.sort(counts)[::-1]
    res = {"slots": int(counts.sum()), "touched": int(np.count_nonzero(counts)), "top16": srt[:16].tolist(),
           "min_nonzero": int(srt[srt > 0].min()), "max_share": round(float(srt[0]) / wl.t, 4)}
    if "zipf_s" in wl.cfg:
        res["zipf_s"] = wl.cfg["zipf_s"]
        res["kl_to_zipf"] = round(fz.kl_to_zipf(counts, wl.cfg["zipf_s"]), 4)
        if res["touched"] >= 128:
            res["slope_ranks_9_128"] = round(fz.slope_of_load(counts), 4)
    return res


def time_steps(torch, wl, steps, warmup, stage_events, graph=True):
    """Wall-clock per step over ``steps`` whole steps (router + forward) run from a HIP
    graph that holds ``per`` consecutive steps (10, 5, 2 or 1, dividing ``steps``), as a
    model's graph holds its layers one after another: the CPU launch cost of the kernels
    and the graph launch itself are then off the per-step clock; bracketed by device
    synchronisation.  ``stage_events``: a second, eager pass of the same number of steps
    with HIP events around each stage (recorded by the library on its stream), for the
    per-kernel averages."""
    lib = wl.lib
    for _ in range(warmup):
        wl.step()
    torch.cuda.synchronize()
    g = None
    per = next(p for p in (10, 5, 2, 1) if steps % p == 0)
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per):
                wl.step()
        # untimed replays: at least the warm-up steps and at least WARM_SECONDS of work, so
        # that clocks have settled when the timed region starts (with only a few warm-up
        # steps the first timed replays ran measurably slower than later ones)
        n, t_w = 0, time.perf_counter()
        while n < max(warmup // per, 1) or time.perf_counter() - t_w < WARM_SECONDS:
            g.replay()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if g is not None:
        for _ in range(steps // per):
            g.replay()
    else:
        for _ in range(steps):
            wl.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stage_ms = {}
    if stage_events:
        evs = []
        for _ in range(steps):
            b = [torch.cuda.Event(enable_timing=True) for _ in lib._lib.STAGES]
            e = [torch.cuda.Event(enable_timing=True) for _ in lib._lib.STAGES]
            for ev in b + e:
                ev.record()  # creates the underlying HIP event; the library re-records it
            evs.append((b, e))
        torch.cuda.synchronize()
        for s in range(steps):
            lib._lib.set_stage_events(*evs[s])
            wl.step()
        torch.cuda.synchronize()
        lib._lib.set_stage_events(None, None)
        used = ["permute", "gate_up", "down", "combine"] if wl.mode == lib.Q4_W4A16 else list(lib._lib.STAGES)
        for name in used:
            si = lib._lib.STAGES.index(name)
            stage_ms[name] = sum(b[si].elapsed_time(e[si]) for b, e in evs) / steps
    del g
    return (t1 - t0) / steps, stage_ms


_FLUSH = []


def flush_caches(torch):
    """Reads 1 GiB (asynchronously, on the current stream), so that nothing of the
    previous step is left in the 256 MB Infinity Cache or the L2s."""
    if not _FLUSH:
        _FLUSH.append(torch.ones(1 << 28, dtype=torch.float32, device="cuda"))
    _FLUSH[0].sum()


def time_cold(torch, wl, steps):
    """Median time of one graph-replayed step that finds neither weights nor activations
    in any cache: a 1 GiB read runs before every replay, outside the events around it."""
    wl.step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wl.step()
    g.replay()
    torch.cuda.synchronize()
    evs = []
    for _ in range(steps):
        flush_caches(torch)
        b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b.record()
        g.replay()
        e.record()
        evs.append((b, e))
    torch.cuda.synchronize()
    ms = sorted(b.elapsed_time(e) for b, e in evs)
    del g
    return ms[len(ms) // 2] * 1e-3


def summarize(wl, sec_per_step, stage_ms, cold_sec=None):
    touched = wl.touched()
    gu_all, dn_all = wl.touched_bytes()
    h, i = wl.cfg["hidden"], wl.cfg["inter"]
    rows = wl.t * (wl.cfg["top_k"] + (1 if wl.layer.shared else 0))
    layer_bytes = gu_all + dn_all
    res = {
        "tokens": wl.t,
        "tokens_per_s": wl.t / sec_per_step,
        "ms_per_step": sec_per_step * 1e3,
        "experts_touched": touched,
        "effective_weight_GBps": layer_bytes / sec_per_step / 1e9,
        "hbm_frac": layer_bytes / sec_per_step / 1e9 / HBM_PEAK_GBS,
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
    }
    if cold_sec is not None:   # every step from HBM (caches flushed before it)
        res["ms_per_step_cold"] = cold_sec * 1e3
        res["hbm_frac_cold"] = layer_bytes / cold_sec / 1e9 / HBM_PEAK_GBS
    load = expert_load(wl)
    if load is not None:
        res["expert_load"] = load
    flops = wl.flops()
    int8 = wl.mode in (wl.lib.Q4_W4A8, wl.lib.Q4_W8A8)
    peak = INT8_PEAK_TOPS if int8 else BF16_PEAK_TFLOPS
    res["mfma_frac"] = flops / sec_per_step / 1e12 / peak
    if "gate_up" in stage_ms:
        act = rows * h * (1 if int8 else 2) + rows * i * (4 if int8 else 2)
        res["gate_up_bytes"] = gu_all + act
        res["gate_up_GBps"] = res["gate_up_bytes"] / (stage_ms["gate_up"] * 1e-3) / 1e9
        res["gate_up_flops"] = 2.0 * rows * 2 * i * h
    return res


def hotness_bits(lib, torch, synth, cfg_name, frac8, calib_tokens=4096):
    """Per-expert widths from routing hit counts of a seeded calibration batch (routed
    by the library's router): the ceil(frac8 * E) most-hit experts in 8 bits."""
    cfg = synth.CONFIGS[cfg_name]
    x = synth.tokens(cfg_name, calib_tokens, device="cuda", salt=7)
    wr, b = synth.router_weights(cfg_name, device="cuda")
    _, ids, _ = lib.moe_route_topk(x, wr, b, cfg["top_k"])
    counts = torch.bincount(ids.reshape(-1).long(), minlength=cfg["experts"]).cpu().tolist()
    return lib.expert_bits_by_hotness(counts, frac8, shared=bool(cfg.get("shared", False)))


def hotness_apex(lib, torch, synth, cfg_name, cold_share=0.25, calib_tokens=4096):
    """APEX widths from hit counts of the same calibration batch: experts hit less than
    cold_share times the even share 2 bits, the others (and the shared expert) 4."""
    cfg = synth.CONFIGS[cfg_name]
    x = synth.tokens(cfg_name, calib_tokens, device="cuda", salt=7)
    wr, b = synth.router_weights(cfg_name, device="cuda")
    _, ids, _ = lib.moe_route_topk(x, wr, b, cfg["top_k"])
    counts = torch.bincount(ids.reshape(-1).long(), minlength=cfg["experts"]).cpu().tolist()
    return lib.expert_bits_apex(counts, 0.0, cold_share, shared=bool(cfg.get("shared", False)))


def hotness_groups(lib, torch, synth, cfg_name, calib_tokens=4096):
    """Per-expert group sizes from routing hit counts of the same calibration batch: the
    top 5 % of the experts 32, experts under a tenth of the even share 256, others 64."""
    cfg = synth.CONFIGS[cfg_name]
    x = synth.tokens(cfg_name, calib_tokens, device="cuda", salt=7)
    wr, b = synth.router_weights(cfg_name, device="cuda")
    _, ids, _ = lib.moe_route_topk(x, wr, b, cfg["top_k"])
    counts = torch.bincount(ids.reshape(-1).long(), minlength=cfg["experts"]).cpu().tolist()
    return lib.expert_groups_by_hotness(counts, 0.05, 0.1, shared=bool(cfg.get("shared", False)))


def cpu_baseline(synth, wl, ntok):
    """The oracle (fp64 NumPy) on the first ``ntok`` tokens of the batch: router + MoE
    forward with the shared expert; expert quantisation (offline) is not timed."""
    import numpy as np
    from oracle import ffn, quant, router
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    x = synth.to_numpy(wl.x[:ntok])
    wr, b = synth.to_numpy(wl.wr), synth.to_numpy(wl.bias) if wl.bias is not None else None
    k = wl.cfg["top_k"]
    # routing of the sample decides which experts the oracle needs (untimed preparation)
    ids0 = router.select_topk(router.logits_fp64(x, wr, b), k)
    need = sorted(set(int(v) for v in ids0.ravel()))
    shared_e = wl.cfg["experts"] if wl.layer.shared else None
    lib = wl.lib
    name, fwd = {lib.Q4_W4A16: ("W4A16", ffn.moe_w4a16), lib.Q4_W4A8: ("W4A8", ffn.moe_w4a8),
                 lib.Q4_W8A8: ("W8A8", ffn.moe_w8a8)}[wl.mode]
    qz = quant.quantize_sym8 if wl.mode == lib.Q4_W8A8 else quant.quantize_sym
    experts = {}
    for e in need + ([shared_e] if shared_e is not None else []):
        g, u, d = synth.expert_weights(wl.cfg_name, e)
        experts[e] = tuple((lambda q: (q[0].astype(np.int64), q[1], None))(qz(synth.to_numpy(m)))
                           for m in (g, u, d))
    # the timed sample is repeated until about 10 s of CPU work have been done
    reps, dt = 0, 0.0
    t0 = time.perf_counter()
    while reps == 0 or dt < 10.0:
        L = router.logits_fp64(x, wr, b)
        ids = router.select_topk(L, k)
        w = router.topk_weights(L, ids)
        out = fwd(x, lambda e: experts[e], ids, w, shared=experts.get(shared_e))
        reps += 1
        dt = time.perf_counter() - t0
    assert np.all(np.isfinite(out))
    return {"value": ntok * reps / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"oracle router + {name} MoE forward (fp64 NumPy) on {ntok} of the {wl.t} tokens "
                      f"({len(need)} routed experts{' + shared' if shared_e is not None else ''}), "
                      f"repeated {reps}x: {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1"}))
        log("bench.py: only --gpus 1 is supported (single-GPU build)")
        return 2
    import torch
    import int4_group_quantized_g128_amd as lib
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    log(f"[bench] building {args.config} layer (T={args.tokens}, {args.mode})")
    wl = Workload(lib, torch, synth, args.config, args.tokens, args.mode)
    log(f"[bench] layer weights {wl.layer.weight_bytes() / 1e9:.3f} GB; timing {args.steps} steps")
    sec, stage_ms = time_steps(torch, wl, args.steps, args.warmup, stage_events=True, graph=not args.no_graph)
    cold = time_cold(torch, wl, min(args.steps, 50)) if not (args.no_graph or args.no_cold) else None
    main_res = summarize(wl, sec, stage_ms, cold)
    log(f"[bench] main: {json.dumps(main_res)}")

    roof = None
    if args.config != "moe256" or args.tokens > 256:   # prefill: the matrix core bounds the kernel
        gu_ms = main_res["stage_ms"]["gate_up"]
        roof = {"kernel": "k_gemm_pf gate/up + SwiGLU (128-row tiles)", "bound": "mfma",
                "achieved": round(main_res["gate_up_flops"] / (gu_ms * 1e-3) / 1e12, 1),
                "peak": INT8_PEAK_TOPS if wl.mode != lib.Q4_W4A16 else BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "traffic": None, "algorithmic_flops_per_launch": main_res["gate_up_flops"], "avg_launch_ms": gu_ms}
        roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    elif "gate_up_GBps" in main_res:
        roof = {"kernel": "k_gemm gate/up + SwiGLU (W4A16, 16-row tiles)", "bound": "hbm",
                "achieved": round(main_res["gate_up_GBps"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(main_res["gate_up_GBps"] / HBM_PEAK_GBS, 4), "traffic": None,
                "algorithmic_bytes_per_launch": main_res["gate_up_bytes"],
                "avg_launch_ms": main_res["stage_ms"]["gate_up"]}

    prof = TRAFFIC_PROFILES.get((args.config, args.tokens, args.mode))
    if roof is not None and prof is not None:
        from int4_group_quantized_g128_amd import profiling
        kv = profiling.read_kv(prof)
        if kv.get("source_hash") == profiling.source_hash():
            roof["profile"] = os.path.relpath(prof, ROOT)
            if "traffic_bytes[gate_up]" in kv:
                roof["traffic"] = int(kv["traffic_bytes[gate_up]"])
            if "avg_us[gate_up]" in kv:
                # the same kernel's average in the committed rocprofv3 kernel trace, and the
                # fraction it gives with the same algorithmic work (frac uses the live average)
                p_ms = float(kv["avg_us[gate_up]"]) * 1e-3
                work = roof.get("algorithmic_bytes_per_launch") or roof.get("algorithmic_flops_per_launch")
                scale = 1e9 if roof["unit"] == "GB/s" else 1e12
                roof["profile_avg_ms"] = round(p_ms, 5)
                roof["profile_frac"] = round(work / (p_ms * 1e-3) / scale / roof["peak"], 4)
            if "mfma_busy_pct[gate_up]" in kv:   # matrix-core busy cycles (rocprofv3 MfmaUtil)
                roof["mfma_busy_pct_counter"] = float(kv["mfma_busy_pct[gate_up]"])
                roof["mfma_frac_counter"] = float(kv["mfma_frac_counter[gate_up]"])

    extra = {}
    if not args.no_extra and args.config == "moe256":
        other = "w4a8" if args.mode == "w4a16" else "w4a16"
        for t, mode in ((1, args.mode), (4096, args.mode), (1, other), (args.tokens, other), (4096, other)):
            if t == args.tokens and mode == args.mode:
                continue
            log(f"[bench] extra moe256 T={t} {mode}")
            wl2 = wl.retoken(synth, t, mode)
            steps = 10 if t > 1000 else 50
            s2, st2 = time_steps(torch, wl2, steps, 3, stage_events=True, graph=not args.no_graph)
            c2 = time_cold(torch, wl2, steps) if not args.no_graph else None
            extra[f"moe256_T{t}_{mode}"] = summarize(wl2, s2, st2, c2)
            del wl2
            torch.cuda.empty_cache()
        for t in (1, 64, 2048):
            log(f"[bench] extra lora8 T={t}")
            lw = LoraWorkload(lib, torch, synth, "lora8", t)
            s4, _ = time_steps(torch, lw, 20 if t > 1000 else 50, 5, stage_events=False, graph=not args.no_graph)
            c4 = time_cold(torch, lw, 20 if t > 1000 else 50) if not args.no_graph else None
            extra[f"lora8_T{t}_w4a16"] = lw.summary(s4, c4)
            del lw
        log("[bench] extra linear 2048x2048 INT4 g128, T=4 (fp16 x, fp32 y)")
        lw = LinearWorkload(lib, torch, synth)
        sl, _ = time_steps(torch, lw, 100, 10, stage_events=False, graph=not args.no_graph)
        cl = time_cold(torch, lw, 100) if not args.no_graph else None
        extra["linear_T4_w4a16"] = lw.summary(sl, cl)
        del lw
        for t in synth.CONFIGS["dense"]["tokens"]:
            log(f"[bench] extra dense 2048/8192 FFN decode T={t}")
            dw = DenseWorkload(lib, torch, synth, t, "w4a16")
            sd, std = time_steps(torch, dw, 100, 10, stage_events=True, graph=not args.no_graph)
            cd = time_cold(torch, dw, 100) if not args.no_graph else None
            extra[f"dense_T{t}_w4a16"] = summarize(dw, sd, std, cd)
            del dw
        m8 = None
        for t in (1, 16, 256):
            log(f"[bench] extra moe8 decode T={t}")
            m8 = Workload(lib, torch, synth, "moe8", t, "w4a16") if m8 is None else m8.retoken(synth, t)
            s8, st8 = time_steps(torch, m8, 100, 10, stage_events=True, graph=not args.no_graph)
            c8 = time_cold(torch, m8, 100) if not args.no_graph else None
            extra[f"moe8_T{t}_w4a16"] = summarize(m8, s8, st8, c8)
        del m8
        for mode in ("w4a8", "w8a8"):
            log(f"[bench] extra moe8 {mode} prefill T=2048")
            w8 = Workload(lib, torch, synth, "moe8_w4a8", 2048, mode)
            s3, st3 = time_steps(torch, w8, 20, 5, stage_events=True, graph=not args.no_graph)
            c3 = time_cold(torch, w8, 20) if not args.no_graph else None
            extra[f"moe8_T2048_{mode}"] = summarize(w8, s3, st3, c3)
            del w8
        log("[bench] extra moe256 mixed widths (top 5 % of experts by hit count in 8 bits), W4A8")
        bits = hotness_bits(lib, torch, synth, "moe256", 0.05)
        mx = Workload(lib, torch, synth, "moe256", args.tokens, "mixed", expert_bits=bits)
        for t in (args.tokens, 4096):
            mt = mx if t == args.tokens else mx.retoken(synth, t)
            s6, st6 = time_steps(torch, mt, 10 if t > 1000 else 50, 3, stage_events=True,
                                 graph=not args.no_graph)
            extra[f"moe256_T{t}_mixed_top5pct_int8"] = dict(summarize(mt, s6, st6), experts_8bit=sum(
                b == 8 for b in bits))
            del mt
        del mx
        torch.cuda.empty_cache()
        log("[bench] extra moe256 APEX widths (experts under a quarter of the even share in 2 bits), W4A8")
        abits = hotness_apex(lib, torch, synth, "moe256")
        aw = Workload(lib, torch, synth, "moe256", args.tokens, "mixed", expert_bits=abits)
        for t in (args.tokens, 4096):
            at = aw if t == args.tokens else aw.retoken(synth, t)
            s9, st9 = time_steps(torch, at, 10 if t > 1000 else 50, 3, stage_events=True, graph=not args.no_graph)
            extra[f"moe256_T{t}_apex_int2"] = dict(summarize(at, s9, st9), experts_2bit=sum(b == 2 for b in abits))
            del at
        del aw
        torch.cuda.empty_cache()
        log("[bench] extra moe256 per-expert group sizes (hit counts: top 5 % 32, cold 256, others 64)")
        groups = hotness_groups(lib, torch, synth, "moe256")
        gw = Workload(lib, torch, synth, "moe256", args.tokens, "w4a16", expert_groups=groups)
        for t, mode in ((args.tokens, "w4a16"), (args.tokens, "w4a8"), (4096, "w4a16"), (4096, "w4a8")):
            gt = gw if (t, mode) == (args.tokens, "w4a16") else gw.retoken(synth, t, mode)
            s7, st7 = time_steps(torch, gt, 10 if t > 1000 else 50, 3, stage_events=True, graph=not args.no_graph)
            extra[f"moe256_T{t}_groups_{mode}"] = dict(summarize(gt, s7, st7), groups={
                str(g): sum(v == g for v in groups) for g in (32, 64, 128, 256)})
            del gt
        del gw
        torch.cuda.empty_cache()
        if args.mode != "w8a8":
            log(f"[bench] extra moe256 W8A8 T={args.tokens}")
            w8 = Workload(lib, torch, synth, "moe256", args.tokens, "w8a8")
            s5, st5 = time_steps(torch, w8, 50, 5, stage_events=True, graph=not args.no_graph)
            extra[f"moe256_T{args.tokens}_w8a8"] = summarize(w8, s5, st5)
            del w8
            torch.cuda.empty_cache()

    if args.copy_calibration:
        n = 512 * 1024 * 1024
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        extra["copy_calibration_bytes"] = n

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {args.cpu_tokens} tokens")
        cpu = cpu_baseline(synth, wl, args.cpu_tokens)

    res = {
        "metric": "tokens/s per MoE layer forward (INT4 g128 experts, router to combine)",
        "value": round(main_res["tokens_per_s"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.mode == "w4a16" else "int8",
        "data": "synthetic",
        "config": {"workload": (f"moe256 {'decode' if args.tokens <= 256 else 'prefill'}: hidden 7168, 256 experts "
                                f"x inter 2048 + 1 shared, top-8, INT4 g128 sym, T={args.tokens}, {args.mode}"
                                if args.config == "moe256" else
                                f"moe8 prefill: hidden 2048, 8 experts x inter 1024, top-2, INT4 g128 sym, 1 % hot "
                                f"channels x10, T={args.tokens}, {args.mode}"),
                   "tokens": args.tokens, "experts_touched": main_res["experts_touched"],
                   "expert_load": main_res.get("expert_load"),
                   "effective_weight_GBps": round(main_res["effective_weight_GBps"], 1),
                   "hbm_frac": round(main_res["hbm_frac"], 4)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "stage_ms": main_res["stage_ms"],
        # the same step with the caches flushed before it (median; 1 GiB read in between)
        "ms_per_step_cold": round(main_res["ms_per_step_cold"], 5) if "ms_per_step_cold" in main_res else None,
        "extra": extra,
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
