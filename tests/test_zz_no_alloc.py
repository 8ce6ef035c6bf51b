"""moe_forward_noalloc (no caller workspace; the library's per-device scratch
array) against moe_forward with a workspace, through the C ABI: bit-identical
outputs on two calls in a row, the second on a smaller batch, in both shared
modes, and the size limit reported as MOE_ERR_WORKSPACE."""

import ctypes

import pytest
import torch

import workloads
from gpu_util import inputs

pytestmark = pytest.mark.gpu

LC = workloads.LayerConfig

CASES = {
    # self-sorted 16-row blocks, routing inside stage 1
    "decode": workloads.CONFIGS["decode_bf16"],
    # sorted 64-row blocks, tiled kernels, a8w8 row quantisation
    "a8w8": LC("noalloc_a8w8", T=200, H=512, E=16, I=256, I_s=256, topk=4, score="sigmoid", n_group=4,
               topk_group=2, fmt="a8w8", gated=False, logits="zipf", zipf_s=1.2),
    # router weights instead of logits: the logits GEMM writes into the scratch
    "router": LC("noalloc_router", T=150, H=512, E=40, I=128, I_s=128, topk=4, fmt="bf16", router_std=0.05),
}


def _smaller(inp, T):
    out = dict(inp)
    for k in ("x", "logits", "x_scale"):
        if out.get(k) is not None:
            out[k] = out[k][:T].contiguous()
    return out


@pytest.mark.parametrize("mode", ["pseudo", "aux"])
@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_workspace_forward(gpu, name, mode):
    import routed_shared_experts_amd as m
    cfg = CASES[name]
    full = inputs(cfg, gpu)
    for T in (cfg.T, cfg.T // 2 + 3):  # second call: a smaller batch
        c = cfg.replace(T=T)
        inp = _smaller(full, T)
        layer = m.MoeLayer(c, inp, shared_mode=mode)
        ref = layer.forward().clone()
        torch.cuda.synchronize()
        got = torch.full_like(layer.out, float("nan"))
        args = m.forward_args(c, layer.inp, got, mode, 0)
        m.moe_forward_noalloc(args, aux_stream=layer.aux_stream, ev_fork=layer.ev_fork.cuda_event,
                              ev_ready=layer.ev_ready.cuda_event)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"{name}/{mode}/T={T}"


def test_noalloc_rejects_requests_beyond_its_scratch(gpu):
    import routed_shared_experts_amd as m
    cfg = workloads.CONFIGS["prefill_bf16"]  # per-pair rows alone need T*k'*H*4 bytes
    inp = inputs(cfg, gpu)
    layer = m.MoeLayer(cfg, inp, shared_mode="pseudo")
    assert layer.ws_bytes > m.MOE_NOALLOC_SCRATCH_BYTES
    st = m.lib().moe_forward_noalloc(ctypes.byref(layer.args), None, None, None, None)
    assert st == m.MOE_ERR_WORKSPACE
