"""The whole step (router + MoE forward) captured in a HIP graph and replayed: every
replay, with eager work of the same library between replays, reproduces the eager
result bit for bit (the kernels are deterministic and the library allocates, clears
and synchronises nothing inside the step).  600 tokens on 64 experts take the router's
split-weight kernels (the weight split runs inside the step)."""
import numpy as np
import pytest
import torch

import synth
from tests.helpers import build_gpu_layer, random_expert_maker, require_gpu

pytestmark = pytest.mark.gpu

H, I, K = 256, 128, 4


@pytest.fixture(scope="module")
def lib():
    require_gpu()
    import int4_group_quantized_g128_amd as lib
    return lib


@pytest.fixture(scope="module")
def layers(lib):
    made = {}

    def get(e):
        if e not in made:
            made[e] = build_gpu_layer(lib, random_expert_maker(31, H, I), e, H, I, K, shared=True)
        return made[e]
    return get


class Step:
    """Preallocated buffers of one (route, forward) step."""

    def __init__(self, lib, layer, t, mode, salt):
        L = lib._lib
        E = layer.num_experts
        self.E = E
        self.lib, self.layer, self.t, self.mode = lib, layer, t, mode
        self.x = synth.normal(synth.stream_key(32, t, salt), (t, H), 1.0, "cuda").to(torch.bfloat16)
        self.wr = synth.normal(synth.stream_key(33), (E, H), 0.05, "cuda")
        self.bias = synth.normal(synth.stream_key(34), (E,), 0.5, "cuda")
        self.logits = torch.empty((t, E), dtype=torch.float32, device="cuda")
        self.ids = torch.empty((t, K), dtype=torch.int32, device="cuda")
        self.w = torch.empty((t, K), dtype=torch.float32, device="cuda")
        self.rws_bytes = int(L.raw.moe_route_workspace_bytes(t, H, E))
        self.rws = torch.empty(max(self.rws_bytes, 1), dtype=torch.uint8, device="cuda")
        self.out = torch.empty((t, H), dtype=torch.bfloat16, device="cuda")
        self.ws_bytes = layer.workspace_bytes(t, mode)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def __call__(self):
        L = self.lib._lib
        raw, P, st = L.raw, L._ptr, L._stream()
        rc = raw.moe_route_topk(P(self.x), P(self.wr), P(self.bias), self.t, H, self.E, K, P(self.logits),
                                P(self.ids), P(self.w), P(self.rws), self.rws_bytes, st)
        assert rc == 0
        rc = raw.moe_int4_ffn_forward(L.ctypes.byref(self.layer.desc), P(self.x), self.t, P(self.ids), P(self.w),
                                      self.mode, P(self.out), P(self.ws), self.ws_bytes, st)
        assert rc == 0


@pytest.mark.parametrize("mode", [0, 1], ids=["w4a16", "w4a8"])
@pytest.mark.parametrize("e,t", [(16, 5), (16, 300), (64, 600)])
def test_graph_replay_matches_eager(lib, layers, mode, e, t):
    layer = layers(e)
    step = Step(lib, layer, t, mode, salt=1)
    other = Step(lib, layer, 2 * t + 3, mode, salt=2)   # eager work between replays
    step()
    torch.cuda.synchronize()
    ref_out, ref_ids, ref_w = step.out.clone(), step.ids.clone(), step.w.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        step.out.zero_()
        step.ids.fill_(-1)
        other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.ids, ref_ids), f"replay {rep}: ids differ"
        assert torch.equal(step.w, ref_w), f"replay {rep}: weights differ"
        assert torch.equal(step.out, ref_out), f"replay {rep}: output differs"
    assert np.isfinite(synth.to_numpy(ref_out)).all()
