"""The layer forward captured into a HIP graph (MoELayerGPU.graph): every
replay, with new tokens copied into the captured input and eager library
work and synchronisations between the replays, must give bitwise the eager
forward's outputs for the same tokens (the workspaces' counters are left at
zero by every call, and no call records a memset).  Covers the decode step
(64-row tiles), a layer with drops and a shared expert, and the fused
combine."""
from __future__ import annotations

import pytest
import torch

from mixture_experts_layer_08_amd.layer import MoELayerGPU, x_to_device
from mixture_experts_layer_08_amd.synth import CONFIGS, MoEConfig, drop_free, make_inputs

from parity_util import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = {
    "decode-64": (CONFIGS[6], {}),
    "decode-16-fused-combine": (drop_free(MoEConfig("g-dec", "bf16", T=16, H=512, I=512, E=8, k=2,
                                                    cf=1.0, batch=16, seq=1, seed=41)),
                                {"fused_combine": True}),
    "drops-shared": (MoEConfig("g-sh", "bf16", T=1001, H=256, I=256, E=8, k=2, cf=0.8,
                               router_bias0=1.0, shared_I=512, seed=42), {}),
    "gumbel-e32": (MoEConfig("g-gum", "bf16", T=900, H=512, I=256, E=32, k=2, cf=1.25,
                             route="gumbel", seq=900, seed=43), {}),
}
OUTS = ("topk_idx", "topk_w", "probs", "slot", "slot_token", "kept", "dropped", "y", "l_aux")


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name):
    cfg, kw = CASES[name]
    log(f"[graph] {name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} {kw}")
    inp = make_inputs(cfg)
    x0 = x_to_device(inp, cfg, DEV)
    graph_layer = MoELayerGPU(cfg, inp, DEV, **kw)
    eager_layer = MoELayerGPU(cfg, inp, DEV, **kw)
    xg = x0.clone()
    g = graph_layer.graph(xg)
    gen = torch.Generator(device="cpu").manual_seed(cfg.seed)
    for rep in range(4):
        # new tokens (bf16 values), the same in both layers
        xn = (torch.randn(x0.shape, generator=gen) * (1.0 + 0.25 * rep)).to(x0.dtype).to(DEV)
        xg.copy_(xn)
        g.replay()
        eager_layer.forward(xn)       # eager library work between the replays
        torch.cuda.synchronize()
        for n in OUTS:
            a, b = getattr(graph_layer.buf, n), getattr(eager_layer.buf, n)
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), f"{name}: replay {rep}: {n} differs from the eager forward"
    log(f"[graph] {name}: 4 replays bitwise equal to the eager forward")
