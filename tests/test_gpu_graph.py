"""HIP-graph capture of the fused layer forward.  moe_forward issues only
kernel launches and event records/waits (no allocation, no memset, no host
synchronisation), so a captured forward must replay to the same bits as an
eager forward.  Each replay follows eager work that rewrites the layer's
inputs in place, so a replay that reused stale results would fail."""

import pytest
import torch

import workloads
from gpu_util import inputs

pytestmark = pytest.mark.gpu

LC = workloads.LayerConfig

CASES = {
    # self-sorted 16-row blocks, routing inside the stage-1 launch (pseudo mode)
    "decode": (workloads.CONFIGS["decode_bf16"], 0),
    # sort launches and the tiled kernels (64-row blocks, persistent stage 2)
    "sorted": (LC("graph_small", T=100, H=256, E=8, I=128, I_s=192, topk=2, fmt="bf16", logits="iid"), 64),
}


@pytest.mark.parametrize("mode", ["pseudo", "aux"])
@pytest.mark.parametrize("case", list(CASES))
def test_graph_replays_match_eager(gpu, case, mode):
    import routed_shared_experts_amd as m

    cfg, block_m = CASES[case]
    base = inputs(cfg, gpu)
    inp = dict(base, x=base["x"].clone(), logits=base["logits"].clone())
    layer = m.MoeLayer(cfg, inp, shared_mode=mode, block_m=block_m)
    layer.forward()
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward()
    torch.cuda.synchronize()

    gen = torch.Generator(device=gpu)
    gen.manual_seed(20261203)
    for r in range(4):
        if r:  # eager work between replays: fresh inputs written in place
            inp["x"].copy_(torch.randn(inp["x"].shape, generator=gen, device=gpu).to(inp["x"].dtype))
            inp["logits"].copy_(torch.randn(inp["logits"].shape, generator=gen, device=gpu))
        graph.replay()
        torch.cuda.synchronize()
        got = layer.out.clone()
        layer.out.zero_()
        layer.forward()
        torch.cuda.synchronize()
        assert torch.equal(got, layer.out), f"{case}/{mode}: replay {r} differs from the eager forward"
