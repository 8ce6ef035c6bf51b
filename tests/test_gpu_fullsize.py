"""Full-size MX layers (MXFP8 and MXFP4 expert weights at the shape the
benchmark times: T = 512, H = 4096, 128 experts of I = 1536, top-8, shared
I_s = 1536), checked stage by stage through the C ABI in the launch
configuration the fused forward picks by itself (automatic block size), in
both shared-expert modes.

Why stage by stage.  The GPU accumulates stage 1 in fp32 and the oracle in
float64; where h sits near a bf16 or e4m3 rounding boundary the two take
neighbouring, equally correct codes, and stage 2 carries a code step times
|W2| into the output.  With 4-bit weights (few, widely spaced magnitudes)
and heavy-tailed outputs one such step can exceed a fixed fraction of the
output RMS, so a single end-to-end tolerance either fails on correct
roundings or is loose enough to let real mistakes through.  The chain below
pins the fused output instead:

1. the fused forward's output is bit-for-bit the output of the step entry
   points (routing, MX quantisation of x, sort, stage 1, stage 2) run with
   the plan the forward uses;
2. every stage-1 row (routed experts, the shared expert's pseudo-expert
   chunks or its dense pass) matches the oracle's intermediate, up to rare
   one-code roundings of near-boundary values;
3. stage 2 with the reduction onto the output matches an oracle stage 2 fed
   the GPU's own intermediate, within the fp32 / 16-bit pair-row arithmetic.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import inputs, run_forward, auto_block_m, compare_mx_h, stage2_reference

pytestmark = pytest.mark.gpu


def _route(m, cfg, W, kt, n_ps, dev):
    T, k = cfg.T, cfg.topk
    ids = torch.empty((T, kt), dtype=torch.int32, device=dev)
    w = torch.empty((T, kt), dtype=torch.float32, device=dev)
    m.moe_route(W["logits"], ids, w, topk=k, bias=W.get("bias"), n_group=cfg.n_group, topk_group=cfg.topk_group,
                group_score_topk=cfg.group_score_topk,
                score=m.MOE_SCORE_SIGMOID if cfg.score == "sigmoid" else m.MOE_SCORE_SOFTMAX,
                renormalize=cfg.renormalize, routed_scaling_factor=cfg.routed_scaling_factor, n_pseudo=n_ps,
                gamma=torch.ones((T,), dtype=torch.float32, device=dev) if n_ps else None)
    return ids, w


def _sort(m, ids, kt, Et, bm, dev):
    T = ids.shape[0]
    cap = m.moe_sort_capacity(T, kt, Et, bm)
    srt = torch.empty((cap,), dtype=torch.int32, device=dev)
    bexp = torch.empty((cap // bm,), dtype=torch.int32, device=dev)
    counts = torch.empty((Et,), dtype=torch.int32, device=dev)
    offs = torch.empty((Et + 1,), dtype=torch.int32, device=dev)
    nblk = torch.empty((4,), dtype=torch.int32, device=dev)
    sb = m.moe_sort_scratch_bytes(T, kt, Et)
    scratch = torch.empty((sb,), dtype=torch.uint8, device=dev) if sb else None
    m.moe_sort_tokens(ids, Et, bm, cap, srt, bexp, counts, offs, nblk, scratch=scratch)
    return cap, srt, bexp, nblk


def _steps(cfg, inp, mode, dev):
    """The fused forward's plan run through the step entry points.  Returns
    the fp32 output and what the checks need from the intermediate."""
    import routed_shared_experts_amd as m
    from routed_shared_experts_amd import _ptr
    from routed_shared_experts_amd.layer import weights_struct, pack_weights

    assert not cfg.gated
    W = dict(inp, **pack_weights(cfg, inp))
    T, H, E, I, Is, k = cfg.T, cfg.H, cfg.E, cfg.I, cfg.I_s, cfg.topk
    n_ps = -(-Is // I) if mode == "pseudo" else 0
    kt, Et = k + n_ps, E + n_ps
    bm = auto_block_m(T * kt / Et)
    ids, w = _route(m, cfg, W, kt, n_ps, dev)
    x = torch.empty((T, H), dtype=torch.uint8, device=dev)
    x_scale = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
    m.moe_quant_mx(W["x"], x, x_scale)
    cap, srt, bexp, nblk = _sort(m, ids, kt, Et, bm, dev)
    h = torch.empty((cap, I), dtype=torch.uint8, device=dev)
    hs = torch.empty((cap, I // 32), dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    counters = torch.zeros((T * (H // 64) + 16,), dtype=torch.int32, device=dev)
    pair_out = torch.empty((T * kt * H,), dtype=torch.float32, device=dev)

    def args():
        a = m.MoeStageArgs()
        a.T, a.H, a.E, a.I, a.I_s, a.n_pseudo, a.k_total = T, H, E, I, Is, n_ps, kt
        a.routed = weights_struct(W["w13"], W["w2"], W.get("w13_scale"), W.get("w2_scale"), cfg.fmt)
        a.shared = weights_struct(W["ws13"], W["ws2"], W.get("ws13_scale"), W.get("ws2_scale"), cfg.fmt)
        a.x, a.x_scale = _ptr(x), _ptr(x_scale)
        return a

    shared = None
    acc = None
    if mode == "aux":   # the dense shared expert: stage 1, then STORE gamma * S(x) as the addend
        dbm = min(auto_block_m(T), 128)
        nb = -(-T // dbm)
        h_sh = torch.empty((nb * dbm, Is), dtype=torch.uint8, device=dev)
        hs_sh = torch.empty((nb * dbm, Is // 32), dtype=torch.uint8, device=dev)
        acc = torch.empty((T, H), dtype=torch.float32, device=dev)
        d = args()
        d.dense, d.block_m, d.max_blocks = 1, dbm, nb
        d.h, d.h_scale = _ptr(h_sh), _ptr(hs_sh)
        d.acc, d.mode = _ptr(acc), m.MOE_STAGE2_STORE
        m.moe_stage1(d)
        m.moe_stage2_accum(d)
        torch.cuda.synchronize()
        shared = (h_sh[:T].cpu().numpy(), hs_sh[:T].cpu().numpy())
    a = args()
    a.dense, a.block_m, a.max_blocks = 0, bm, cap // bm
    a.sorted_pair_ids, a.block_expert, a.num_blocks = _ptr(srt), _ptr(bexp), _ptr(nblk)
    a.h, a.h_scale = _ptr(h), _ptr(hs)
    a.pair_w, a.acc = _ptr(w), _ptr(acc)
    a.pair_out, a.out, a.out_dtype = _ptr(pair_out), _ptr(out), m.MOE_F32
    a.mode, a.counters, a.expected_arrivals = m.MOE_STAGE2_ACCUMULATE, _ptr(counters), kt
    m.moe_stage1(a)
    torch.cuda.synchronize()
    hq, hsc = h.cpu().numpy(), hs.cpu().numpy()
    m.moe_stage2_accum(a)
    torch.cuda.synchronize()
    return dict(out=out, srt=srt.cpu().numpy(), ids=ids.cpu().numpy(), w=w.cpu().numpy().astype(np.float64),
                h=hq, hs=hsc, kt=kt, n_ps=n_ps, bm=bm, shared=shared)


@pytest.mark.parametrize("mode", ["pseudo", "aux"])
@pytest.mark.parametrize("name", ["mxfp8", "mxfp4"])
def test_full_size_mx_layer_stage_by_stage(gpu, name, mode):
    import routed_shared_experts_amd as m
    cfg = workloads.CONFIGS[name]
    inp = inputs(cfg, gpu)
    print(f"case {name}/{mode}", flush=True)
    st = _steps(cfg, inp, mode, gpu)

    # 1. the fused forward (automatic plan) is the step chain, bit for bit
    fused, layer = run_forward(cfg, inp, mode, out_dtype=m.MOE_F32)
    n_diff = int((fused != st["out"]).sum())
    assert n_diff == 0, f"{name}/{mode}: {n_diff} outputs differ between the fused forward and its steps"

    # 2. stage 1 against the oracle, every row
    host = workloads.to_host(inp, lazy_weights=True)
    T, E, I, k, kt = cfg.T, cfg.E, cfg.I, cfg.topk, st["kt"]
    srt, flat = st["srt"], st["ids"].reshape(-1)
    P = T * kt
    tot = np.zeros(4, dtype=np.int64)
    valid = np.nonzero(srt < P)[0]
    for e in range(E + st["n_ps"]):
        slots = valid[flat[srt[valid]] == e]
        if slots.size == 0:
            continue
        toks = srt[slots] // kt
        if e < E:
            ref = oracle.stage1_reference(host, cfg, e, toks)["h"]
        else:
            c = e - E
            ref = oracle.stage1_reference(host, cfg, E, toks)["h"][:, c * I:(c + 1) * I]
        tot += compare_mx_h(st["h"][slots][:, :ref.shape[1]], st["hs"][slots][:, :ref.shape[1] // 32], ref,
                            f"{name} expert {e}")
    if st["shared"] is not None:
        ref = oracle.stage1_reference(host, cfg, E, np.arange(T))["h"]
        tot += compare_mx_h(st["shared"][0], st["shared"][1], ref, f"{name} dense shared")
    rate = tot[1] / tot[0]
    print(f"stage 1 {name}/{mode}/bm{st['bm']}: {tot[1]} of {tot[0]} values one code off (rate {rate:.2e}); "
          f"{tot[3]} of {tot[2]} MX blocks with a scale one step off", flush=True)
    assert rate <= 1e-2 and tot[3] <= 0.01 * tot[2]

    # 3. stage 2 and the reduction against the oracle on the GPU's intermediate
    h_vals = oracle.mx_dequantize(st["hs"], st["h"])
    shared = None
    if st["shared"] is not None:
        shared = (oracle.mx_dequantize(st["shared"][1], st["shared"][0]), np.ones(T), np.ones(T))
    y = stage2_reference(cfg, host, srt, st["ids"], st["w"], h_vals, np.ones(h_vals.shape[0]), kt, shared=shared)
    got = st["out"].cpu().numpy().astype(np.float64)
    rms = np.sqrt((y ** 2).mean())
    rel = np.abs(got - y).max() / rms
    # fp32 accumulation and the 16-bit pair rows: each of the kt terms within
    # 2^-13 of its tile's largest magnitude (at most max |y| here)
    bound = kt * 2.0 ** -13 * np.abs(y).max() / rms + 1e-4
    print(f"stage 2 {name}/{mode}: max|err|/rms={rel:.3e} (bound {bound:.3e}, max|y|/rms "
          f"{np.abs(y).max() / rms:.1f})", flush=True)
    assert rel <= bound
