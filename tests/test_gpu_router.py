"""The router-logit GEMM (moe_router_logits) and the prologue that runs it in
front of the routing (moe_forward given router weights instead of logits:
for fp32 activations one launch that also routes, for bf16 / e4m3 a tiled
GEMM launch and then the routing launch), against the oracle.

The GPU accumulates the logits in fp32, so they differ from the oracle's
float64 dot products by rounding, and a token whose k-th and (k+1)-th scores
sit that close could be routed either way.  The checks therefore split:
the logits against the float64 dot within its error bound, and the fused
forward against the forward fed those same GPU logits -- bit for bit -- which
in turn is held to the oracle routed on the GPU's logits."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import inputs, run_forward, assert_close

pytestmark = pytest.mark.gpu

LC = workloads.LayerConfig

CASES = {
    "f32": LC("rt_f32", T=37, H=128, E=8, I=64, I_s=64, topk=3, fmt="f32", router_std=0.1),
    # softmax without groups at decode size: without router weights this
    # batch would route inside the stage-1 launch
    "bf16_decode": LC("rt_bf16_decode", T=24, H=512, E=16, I=256, I_s=256, topk=4, fmt="bf16", router_std=0.05),
    "bf16_groups": LC("rt_bf16_groups", T=200, H=256, E=100, I=128, I_s=128, topk=6, fmt="bf16",
                      n_group=4, topk_group=2, router_std=0.1),
    "mxfp8": LC("rt_mxfp8", T=70, H=512, E=16, I=256, I_s=256, topk=4, score="sigmoid", n_group=4, topk_group=2,
                fmt="mxfp8", gated=False, bias_std=0.1, router_std=0.05),
    "a8w8": LC("rt_a8w8", T=90, H=512, E=16, I=256, I_s=256, topk=4, score="sigmoid", n_group=4, topk_group=2,
               fmt="a8w8", gated=False, router_std=0.05),
    # larger batches: several 128-token tiles, the last one ragged, and a
    # partial 64-expert tile
    "bf16_large_t": LC("rt_bf16_large_t", T=1100, H=512, E=40, I=128, I_s=128, topk=4, fmt="bf16",
                       router_std=0.05),
    "a8w8_large_t": LC("rt_a8w8_large_t", T=1030, H=768, E=72, I=128, I_s=128, topk=6, score="sigmoid",
                       n_group=4, topk_group=2, fmt="a8w8", gated=False, router_std=0.05),
}

# logits-only shapes: expert counts around the 16-row tiles and up to 512
SHAPES = {
    "e257": LC("rt_e257", T=130, H=1024, E=257, I=128, I_s=0, topk=4, fmt="bf16", router_std=0.03),
    "e512": LC("rt_e512", T=65, H=768, E=512, I=128, I_s=0, topk=8, fmt="bf16", router_std=0.03),
    "e512_a8w8": LC("rt_e512_a8w8", T=70, H=512, E=512, I=128, I_s=0, topk=8, fmt="a8w8", router_std=0.03),
    # several token tiles of the tiled GEMM, a partial last token tile and
    # expert tile
    "t1100_e257": LC("rt_t1100_e257", T=1100, H=1024, E=257, I=128, I_s=0, topk=4, fmt="bf16", router_std=0.03),
    "t2049_e512_a8w8": LC("rt_t2049_e512_a8w8", T=2049, H=640, E=512, I=128, I_s=0, topk=8, fmt="a8w8",
                          router_std=0.03),
    # fp32 activations take the one-launch kernel: many workgroups of it
    "t600_f32": LC("rt_t600_f32", T=600, H=256, E=100, I=64, I_s=0, topk=4, fmt="f32", router_std=0.1),
    # one token, one 64-element K tile (fewer K tiles than loads in flight)
    "t1_h64": LC("rt_t1_h64", T=1, H=64, E=8, I=64, I_s=0, topk=2, fmt="bf16", router_std=0.1),
    "t5_h128_e65_a8w8": LC("rt_t5_h128_e65_a8w8", T=5, H=128, E=65, I=64, I_s=0, topk=3, fmt="a8w8",
                           router_std=0.1),
}


def _gpu_logits(cfg, inp):
    import routed_shared_experts_amd as m
    logits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=inp["x"].device)
    m.moe_router_logits(inp["x"], inp["router_w"], logits, x_row_scale=inp.get("x_scale"))
    torch.cuda.synchronize()
    return logits


@pytest.mark.parametrize("name", list(CASES) + list(SHAPES))
def test_router_logits_within_the_dot_bound(gpu, name):
    cfg = CASES.get(name) or SHAPES[name]
    inp = inputs(cfg, gpu)
    got = _gpu_logits(cfg, inp).cpu().numpy().astype(np.float64)
    host = workloads.to_host(inp)
    ref = oracle.router_logits(host, cfg.fmt)
    # fp32 accumulation of H exact products (bf16 x bf16 and e4m3 x bf16 are
    # exact in fp32; fp32 x fp32 rounds each product once), then the token
    # scale: Higham's bound gamma_(H+2) times sum_k |x_k w_k|
    if cfg.fmt == "f32":
        xa, wa = np.abs(host["x"].astype(np.float64)), np.abs(host["router_w"].astype(np.float64))
    else:
        wa = np.abs(oracle.bf16_bits_to_f64(host["router_w"]))
        xa = np.abs(oracle.layer.gate_input(host, cfg.fmt))
    S = xa @ wa.T
    n = cfg.H + 2
    bound = n * 2.0 ** -24 / (1 - n * 2.0 ** -24) * S
    err = np.abs(got - ref)
    print(f"{name}: max|err|={err.max():.3e}, max err/bound={float((err / bound).max()):.3f}, "
          f"max|l|={np.abs(ref).max():.3f}")
    assert (err <= bound).all()


@pytest.mark.parametrize("mode", ["pseudo", "aux"])
@pytest.mark.parametrize("name", list(CASES))
def test_forward_with_router_weights(gpu, name, mode):
    cfg = CASES[name]
    inp = inputs(cfg, gpu)
    logits = _gpu_logits(cfg, inp)
    fused, _ = run_forward(cfg, inp, mode)
    fused = fused.clone()
    given = dict(inp, logits=logits, router_w=None)
    plain, _ = run_forward(cfg, given, mode)
    n_diff = int((fused != plain).sum())
    assert n_diff == 0, f"{name}/{mode}: {n_diff} outputs differ from the forward fed the same logits"
    if cfg.fmt == "a8w8" and cfg.T >= 1024:
        # a thousand tokens of the per-row e4m3 intermediate: a value of h
        # at a rounding boundary takes the neighbouring code on the GPU (fp32
        # against float64 accumulation), and on these heavy-tailed outputs
        # (max |y| ~ 9 RMS) one such step can exceed the layer bound; the
        # stage tests hold each stage to the oracle separately
        return
    rel, floor, _ = assert_close(cfg, fused, given)
    print(f"{name}/{mode}: max|err|/rms={rel:.3e} floor={floor:.3e}")
