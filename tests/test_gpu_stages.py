"""Parity of the layer built from the step entry points alone, through the C
ABI: shared_gate_dot, moe_route, moe_quant_mx, moe_sort_tokens, moe_stage1 and
moe_stage2_accum, with no moe_forward call.  Two arrangements of the shared
expert: as always-selected pseudo-experts of the routed GEMM (route with
pseudo slots, one ACCUMULATE stage 2), and as a dense stage 1 plus a STORE
stage 2 whose output is the addend of the routed ACCUMULATE stage 2.  Every
format, with 16-row blocks (one-wave kernels fed by the sort) and 64-row
blocks (tiled kernels; the LDS-staged fallback for f32), compared on every
output with the oracle's layer."""

import ctypes

import numpy as np

import pytest
import torch

import workloads
from gpu_util import inputs, assert_close, stage2_reference

pytestmark = pytest.mark.gpu

LC = workloads.LayerConfig

CASES = {
    "f32": LC("steps_f32", T=37, H=128, E=8, I=64, I_s=64, topk=3, fmt="f32", logits="iid"),
    "bf16": LC("steps_bf16", T=100, H=256, E=8, I=128, I_s=128, topk=2, fmt="bf16", logits="iid"),
    "mxfp8": LC("steps_mxfp8", T=70, H=512, E=16, I=256, I_s=256, topk=4, score="sigmoid", n_group=4,
                topk_group=2, routed_scaling_factor=2.5, fmt="mxfp8", gated=False, bias_std=0.1),
    "a8w8": LC("steps_a8w8", T=90, H=512, E=16, I=256, I_s=256, topk=4, score="sigmoid", n_group=4,
               topk_group=2, fmt="a8w8", gated=False, logits="zipf", zipf_s=1.2),
    "mxfp4": LC("steps_mxfp4", T=70, H=512, E=16, I=256, I_s=256, topk=4, score="sigmoid", n_group=4,
                topk_group=2, fmt="mxfp4", gated=False, bias_std=0.1),
    "bias_gelu_bf16": LC("steps_bias_gelu_bf16", T=100, H=256, E=8, I=128, I_s=256, topk=2, fmt="bf16",
                         logits="iid", bias13_std=0.2, bias2_std=0.01, activation="gelu_tanh"),
}

DENSE_BM = 64


def _h_buffers(fmt, rows, width, dev):
    """Stage-1 output storage: values (a8w8: bf16, quantised in place by
    stage 2) and their scales (MX: e8m0 per 32; a8w8: fp32 row max, zero)."""
    if fmt == "f32":
        return torch.empty((rows, width), dtype=torch.float32, device=dev), None
    if fmt == "bf16":
        return torch.empty((rows, width), dtype=torch.bfloat16, device=dev), None
    if fmt in ("mxfp8", "mxfp4"):
        return (torch.empty((rows, width), dtype=torch.uint8, device=dev),
                torch.empty((rows, width // 32), dtype=torch.uint8, device=dev))
    return (torch.empty((rows, width), dtype=torch.bfloat16, device=dev),
            torch.zeros((rows,), dtype=torch.float32, device=dev))


def run_steps(cfg, inp, mode, block_m, dev):
    import routed_shared_experts_amd as m
    from routed_shared_experts_amd import _ptr
    from routed_shared_experts_amd.layer import FORMATS, weights_struct, pack_weights

    W = dict(inp, **pack_weights(cfg, inp))
    _, _, _, odt = FORMATS[cfg.fmt]
    T, H, E, I, Is, k = cfg.T, cfg.H, cfg.E, cfg.I, cfg.I_s, cfg.topk
    n_ps = -(-Is // I) if mode == "pseudo" else 0
    kt = k + n_ps
    keep = []  # tensors whose pointers the launches use

    # gate and routing (pseudo slots carry the gate)
    gamma = torch.ones((T,), dtype=torch.float32, device=dev)
    if cfg.gated:
        m.shared_gate_dot(W["x"], W["gate_w"], gamma)
    ids = torch.empty((T, kt), dtype=torch.int32, device=dev)
    w = torch.empty((T, kt), dtype=torch.float32, device=dev)
    m.moe_route(W["logits"], ids, w, topk=k, bias=W.get("bias"), n_group=cfg.n_group, topk_group=cfg.topk_group,
                group_score_topk=cfg.group_score_topk,
                score=m.MOE_SCORE_SIGMOID if cfg.score == "sigmoid" else m.MOE_SCORE_SOFTMAX,
                renormalize=cfg.renormalize, routed_scaling_factor=cfg.routed_scaling_factor, n_pseudo=n_ps,
                gamma=gamma if n_ps else None)

    # the GEMMs' activation input
    if cfg.fmt in ("mxfp8", "mxfp4"):
        xq = torch.empty((T, H), dtype=torch.uint8, device=dev)
        xs = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
        m.moe_quant_mx(W["x"], xq, xs)
        x, x_scale = xq, xs
    else:
        x, x_scale = W["x"], W.get("x_scale")

    def base_args():
        a = m.MoeStageArgs()
        a.T, a.H, a.E, a.I, a.I_s = T, H, E, I, Is
        a.routed = weights_struct(W["w13"], W["w2"], W.get("w13_scale"), W.get("w2_scale"), cfg.fmt,
                                  W.get("b13"), W.get("b2"))
        a.shared = weights_struct(W["ws13"], W["ws2"], W.get("ws13_scale"), W.get("ws2_scale"), cfg.fmt,
                                  W.get("bs13"), W.get("bs2"))
        a.x, a.x_scale = _ptr(x), _ptr(x_scale)
        a.activation = m.ACTIVATIONS[cfg.activation]
        return a

    out = torch.empty((T, H), dtype=torch.float32 if odt == m.MOE_F32 else torch.bfloat16, device=dev)
    acc = None
    if mode == "aux":
        # dense shared expert: stage 1, then STORE of gamma * S(x) into the addend
        acc = torch.empty((T, H), dtype=torch.float32, device=dev)
        nb = -(-T // DENSE_BM)
        hd, hds = _h_buffers(cfg.fmt, nb * DENSE_BM, Is, dev)
        keep += [hd, hds]
        d = base_args()
        d.n_pseudo, d.k_total = 0, 1
        d.dense, d.block_m, d.max_blocks = 1, DENSE_BM, nb
        d.h, d.h_scale = _ptr(hd), _ptr(hds)
        d.gamma = _ptr(gamma) if cfg.gated else None
        d.acc = _ptr(acc)
        d.mode = m.MOE_STAGE2_STORE
        m.moe_stage1(d)
        m.moe_stage2_accum(d)

    # routed (and pseudo) experts: sort, stage 1, ACCUMULATE stage 2
    Et = E + n_ps
    cap = m.moe_sort_capacity(T, kt, Et, block_m)
    sorted_ = torch.empty((cap,), dtype=torch.int32, device=dev)
    bexp = torch.empty((cap // block_m,), dtype=torch.int32, device=dev)
    counts = torch.empty((Et,), dtype=torch.int32, device=dev)
    offsets = torch.empty((Et + 1,), dtype=torch.int32, device=dev)
    nblk = torch.empty((4,), dtype=torch.int32, device=dev)
    sb = m.moe_sort_scratch_bytes(T, kt, Et)
    scratch = torch.empty((sb,), dtype=torch.uint8, device=dev) if sb else None
    m.moe_sort_tokens(ids, Et, block_m, cap, sorted_, bexp, counts, offsets, nblk, scratch=scratch)
    h, hs = _h_buffers(cfg.fmt, cap, I, dev)
    counters = torch.zeros((T * (H // 64) + 16,), dtype=torch.int32, device=dev)  # moe_stage2_counters(T, H)
    pair_out = torch.empty((T * kt * H,), dtype=torch.float32, device=dev)
    a = base_args()
    a.n_pseudo, a.k_total = n_ps, kt
    a.dense, a.block_m, a.max_blocks = 0, block_m, cap // block_m
    a.sorted_pair_ids, a.block_expert, a.num_blocks = _ptr(sorted_), _ptr(bexp), _ptr(nblk)
    a.h, a.h_scale = _ptr(h), _ptr(hs)
    a.pair_w = _ptr(w)
    a.acc = _ptr(acc)
    a.pair_out, a.out, a.out_dtype = _ptr(pair_out), _ptr(out), odt
    a.mode, a.counters, a.expected_arrivals = m.MOE_STAGE2_ACCUMULATE, _ptr(counters), kt
    m.moe_stage1(a)
    m.moe_stage2_accum(a)
    torch.cuda.synchronize()
    del keep
    return out


@pytest.mark.parametrize("block_m", [16, 64])
@pytest.mark.parametrize("mode", ["pseudo", "aux"])
@pytest.mark.parametrize("name", list(CASES))
def test_layer_from_step_entry_points(gpu, name, mode, block_m):
    cfg = CASES[name]
    inp = inputs(cfg, gpu)
    out = run_steps(cfg, inp, mode, block_m, gpu)
    rel, floor, _ = assert_close(cfg, out, inp)
    print(f"steps {name}/{mode}/bm{block_m}: max|err|/rms={rel:.3e} floor={floor:.3e}")


def test_stage2_mode_checks(gpu):
    """moe_stage2_accum's mode checks: STORE needs the dense problem and an
    addend, ACCUMULATE the sorted one (no launch on either error)."""
    import routed_shared_experts_amd as m
    from routed_shared_experts_amd import _ptr
    from routed_shared_experts_amd.layer import weights_struct, pack_weights

    cfg = CASES["bf16"]
    inp = inputs(cfg, gpu)
    W = dict(inp, **pack_weights(cfg, inp))
    h, _ = _h_buffers("bf16", 2 * DENSE_BM, cfg.I_s, gpu)
    a = m.MoeStageArgs()
    a.T, a.H, a.E, a.I, a.I_s, a.k_total = cfg.T, cfg.H, cfg.E, cfg.I, cfg.I_s, 1
    a.routed = weights_struct(W["w13"], W["w2"], None, None, "bf16")
    a.shared = weights_struct(W["ws13"], W["ws2"], None, None, "bf16")
    a.x, a.h = _ptr(W["x"]), _ptr(h)
    a.dense, a.block_m, a.max_blocks = 1, DENSE_BM, 2
    a.mode = m.MOE_STAGE2_STORE
    assert m.lib().moe_stage2_accum(ctypes.byref(a), None) == m.MOE_ERR_INVALID_ARG  # no addend
    a.mode = m.MOE_STAGE2_ACCUMULATE
    assert m.lib().moe_stage2_accum(ctypes.byref(a), None) == m.MOE_ERR_UNSUPPORTED  # dense + ACCUMULATE



# ---- stage 2 on the GPU's own stage-1 output ---------------------------------

BIG = {
    # tokens enough for 256-row blocks with several full ones per expert, and
    # outputs with a heavy tail (max |y| about 9x their RMS)
    "big_a8w8": LC("big_a8w8", T=1200, H=512, E=8, I=256, I_s=256, topk=2, score="sigmoid", fmt="a8w8",
                   gated=False, logits="zipf", zipf_s=1.2),
    "big_bf16": LC("big_bf16", T=1200, H=512, E=8, I=256, I_s=256, topk=2, fmt="bf16", logits="zipf", zipf_s=1.2),
    "big_mxfp8": LC("big_mxfp8", T=1200, H=512, E=8, I=256, I_s=256, topk=2, score="sigmoid",
                    fmt="mxfp8", gated=False, bias_std=0.1),
    "big_mxfp4": LC("big_mxfp4", T=1200, H=512, E=8, I=256, I_s=256, topk=2, score="sigmoid",
                    fmt="mxfp4", gated=False, bias_std=0.1),
}


@pytest.mark.parametrize("block_m", [16, 64, 256])
@pytest.mark.parametrize("name", list(BIG))
def test_stage2_against_oracle_on_the_gpus_intermediate(gpu, name, block_m):
    """Stage 2 and the reduction onto the output against an oracle stage 2
    that dequantises the same fp8 values the GPU quantised in stage 1 (the
    intermediate as stored: bf16, MX codes + scales, or bf16 rows that stage
    2 quantises per row), pseudo-expert shared mode.  On these heavy-tailed
    outputs a per-row fp8 quantisation of h that lands one step off the
    oracle's (fp32 against fp64 accumulation in stage 1) moves the output by
    a code step times |o|, so the layer-level error can exceed the bound;
    stage 1 is held to the oracle separately (its intermediate test)."""
    import oracle
    import routed_shared_experts_amd as m
    from routed_shared_experts_amd import _ptr
    from routed_shared_experts_amd.layer import FORMATS, weights_struct, pack_weights

    cfg = BIG[name]
    if cfg.fmt == "mxfp4" and block_m == 256:
        pytest.skip("256-row blocks: the LDS-staged kernels take no e2m1 weights")
    inp = inputs(cfg, gpu)
    dev = gpu
    W = dict(inp, **pack_weights(cfg, inp))
    T, H, E, I, Is, k = cfg.T, cfg.H, cfg.E, cfg.I, cfg.I_s, cfg.topk
    n_ps = -(-Is // I)
    kt = k + n_ps
    ids = torch.empty((T, kt), dtype=torch.int32, device=dev)
    w = torch.empty((T, kt), dtype=torch.float32, device=dev)
    m.moe_route(W["logits"], ids, w, topk=k, bias=W.get("bias"), n_group=cfg.n_group, topk_group=cfg.topk_group,
                score=m.MOE_SCORE_SIGMOID if cfg.score == "sigmoid" else m.MOE_SCORE_SOFTMAX,
                routed_scaling_factor=cfg.routed_scaling_factor, n_pseudo=n_ps,
                gamma=torch.ones((T,), dtype=torch.float32, device=dev))
    if cfg.fmt in ("mxfp8", "mxfp4"):
        x = torch.empty((T, H), dtype=torch.uint8, device=dev)
        x_scale = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
        m.moe_quant_mx(W["x"], x, x_scale)
    else:
        x, x_scale = W["x"], W.get("x_scale")
    Et = E + n_ps
    cap = m.moe_sort_capacity(T, kt, Et, block_m)
    srt = torch.empty((cap,), dtype=torch.int32, device=dev)
    bexp = torch.empty((cap // block_m,), dtype=torch.int32, device=dev)
    counts = torch.empty((Et,), dtype=torch.int32, device=dev)
    offs = torch.empty((Et + 1,), dtype=torch.int32, device=dev)
    nblk = torch.empty((4,), dtype=torch.int32, device=dev)
    sb = m.moe_sort_scratch_bytes(T, kt, Et)
    scratch = torch.empty((sb,), dtype=torch.uint8, device=dev) if sb else None
    m.moe_sort_tokens(ids, Et, block_m, cap, srt, bexp, counts, offs, nblk, scratch=scratch)
    h, hs = _h_buffers(cfg.fmt, cap, I, dev)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    counters = torch.zeros((T * (H // 64) + 16,), dtype=torch.int32, device=dev)
    pair_out = torch.empty((T * kt * H,), dtype=torch.float32, device=dev)
    a = m.MoeStageArgs()
    a.T, a.H, a.E, a.I, a.I_s, a.n_pseudo, a.k_total = T, H, E, I, Is, n_ps, kt
    a.routed = weights_struct(W["w13"], W["w2"], W.get("w13_scale"), W.get("w2_scale"), cfg.fmt)
    a.shared = weights_struct(W["ws13"], W["ws2"], W.get("ws13_scale"), W.get("ws2_scale"), cfg.fmt)
    a.x, a.x_scale = _ptr(x), _ptr(x_scale)
    a.dense, a.block_m, a.max_blocks = 0, block_m, cap // block_m
    a.sorted_pair_ids, a.block_expert, a.num_blocks = _ptr(srt), _ptr(bexp), _ptr(nblk)
    a.h, a.h_scale = _ptr(h), _ptr(hs)
    a.pair_w = _ptr(w)
    a.pair_out, a.out, a.out_dtype = _ptr(pair_out), _ptr(out), m.MOE_F32
    a.mode, a.counters, a.expected_arrivals = m.MOE_STAGE2_ACCUMULATE, _ptr(counters), kt
    m.moe_stage1(a)
    torch.cuda.synchronize()
    # the intermediate as stage 2 will read it
    if cfg.fmt == "bf16":
        h_vals = oracle.bf16_bits_to_f64(h.view(torch.int16).cpu().numpy().view(np.uint16))
        h_scale = np.ones(cap)
    elif cfg.fmt in ("mxfp8", "mxfp4"):
        h_vals = oracle.mx_dequantize(hs.cpu().numpy(), h.cpu().numpy())
        h_scale = np.ones(cap)
    else:
        hb = oracle.bf16_bits_to_f64(h.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float32)
        sc, q = oracle.row_quantize_e4m3(hb)
        h_vals, h_scale = oracle.e4m3_decode(q), sc.astype(np.float64)
    m.moe_stage2_accum(a)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    y = stage2_reference(cfg, workloads.to_host(inp), srt.cpu().numpy(), ids.cpu().numpy(),
                         w.cpu().numpy().astype(np.float64), h_vals, h_scale, kt)
    rms = np.sqrt((y ** 2).mean())
    rel = np.abs(got - y).max() / rms
    print(f"stage 2 on the GPU's intermediate {name}/bm{block_m}: max|err|/rms={rel:.3e} "
          f"(max|y|/rms {np.abs(y).max() / rms:.1f})")
    # fp32 accumulation, and the 16-bit block-scaled pair rows of the tiled
    # kernels: each of the kt terms within 2^-13 of its tile's largest
    # magnitude, at most max |y| here
    bound = kt * 2.0 ** -13 * np.abs(y).max() / rms + 1e-4
    assert rel <= bound, (rel, bound)
