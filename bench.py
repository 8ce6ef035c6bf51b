"""Benchmark of the fused routed + shared-expert MoE layer forward on one MI355X.

One step = one whole layer forward (routing + gate dot + sort + stage 1 +
stage 2 with the shared-expert addend) over one batch of seeded synthetic
inputs already resident in HBM.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload a8w8_large]
                    [--mode auto|pseudo|aux|best] [--graph] [--router] [--no-cpu-baseline]
                    [--copy-calibration MIB]

Per-kernel durations come from HIP events that the layer records between its
launches on every TIMING_EVERY-th step of the timed region (an event record
costs a few microseconds, so recording them on every step would slow the step
being measured).  --copy-calibration runs plain device copies of a known size
after the timed region, for scaling the HBM byte counters of a profiler run.
"""

import hashlib

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s and achieved TFLOPS (% MFMA peak) / GB/s (% HBM) on 1 GPU"
HBM_PEAK_GBS = 8000.0
# mxfp4: e2m1 weights against e4m3 activations run at the fp8 rate
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3, "mxfp8": 5000.0, "mxfp4": 5000.0, "a8w8": 5000.0}
DTYPE_NAME = {"f32": "f32", "bf16": "bf16", "mxfp8": "mxfp8-e4m3", "mxfp4": "mxfp4-e2m1-w/mxfp8-a",
              "a8w8": "fp8-e4m3"}
TIMING_EVERY = 8
N_EVENTS = 7  # timing events the layer takes (prologue and sort spans, each GEMM kernel's start and end)
# sources of the GEMM kernels: a traffic figure in profiles/ holds only while
# the hash of the sources of the kernel it was measured on is unchanged
# (16-row one-wave kernels at decode sizes, the tiled kernels otherwise)
KERNEL_SOURCES = {
    "wave": ["gemm_wave.hip", "gemm_common.hpp", "common.hpp", "kernels.hpp"],
    "tile": ["gemm_tile.hip", "gemm_lds.hip", "tile_common.hpp", "gemm.hip", "gemm_common.hpp", "common.hpp",
             "kernels.hpp"],
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="a8w8_large")
    ap.add_argument("--mode", default="best", choices=["auto", "pseudo", "aux", "best"])
    ap.add_argument("--copies", type=int, default=0, help="weight copies rotated per step (0 = auto)")
    ap.add_argument("--block-m", type=int, default=0, help="rows per sorted block (0 = automatic)")
    ap.add_argument("--graph", action="store_true", help="time HIP-graph replays of the forward")
    ap.add_argument("--router", action="store_true",
                    help="give the layer its router projection (N(0, 1/H) weights) instead of logits, so the "
                         "router GEMM runs in the routing launch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="MIB",
                    help="after timing, copy MIB MiB device-to-device 4 times (profiler counter calibration)")
    return ap.parse_args()


def kernel_sources_sha256(family):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, "routed_shared_experts_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, stage):
    """HBM bytes per launch of the given GEMM stage from the committed profiler
    summary of this workload (FETCH_SIZE + WRITE_SIZE, each scaled by a plain
    copy's reading), or None when there is none or the kernel sources changed
    since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_{stage}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    fam = kv.get("kernel_family", "wave")
    if fam not in KERNEL_SOURCES or kv.get("kernel_sources_sha256") != kernel_sources_sha256(fam):
        return None
    try:
        return float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic(cfg, ids, m_pseudo):
    """Algorithmic FLOPs and bytes of the layer, of stage 1 and of stage 2
    (each stage: its weights once, its activation input once, its output once;
    the shared expert's rows count in the stages when it runs as pseudo-experts)."""
    import workloads
    bw = workloads.bytes_per_weight(cfg.fmt)
    bx = {"f32": 4, "bf16": 2, "mxfp8": 2, "mxfp4": 2, "a8w8": 1}[cfg.fmt]
    bh = {"f32": 4, "bf16": 2, "mxfp8": 1 + 1 / 32, "mxfp4": 1 + 1 / 32, "a8w8": 1}[cfg.fmt]
    bo = 4 if cfg.fmt == "f32" else 2
    T, H, I, Is, k = cfg.T, cfg.H, cfg.I, cfg.I_s, cfg.topk
    P = T * k
    active = int((np.bincount(ids.reshape(-1), minlength=cfg.E)[:cfg.E] > 0).sum())
    flops = 6.0 * H * I * P + 6.0 * H * Is * T + (2.0 * H * T if cfg.gated else 0.0)
    w_routed = active * 3.0 * H * I * bw
    w_shared = 3.0 * H * Is * bw if Is else 0.0
    # active routed weights once, shared weights once, x once, out once, logits,
    # and the stage-1 output written and read once (routed and shared)
    byt = (w_routed + w_shared + T * H * bx + T * H * bo + T * cfg.E * 4
           + 2.0 * P * I * bh + 2.0 * T * Is * bh)
    # stage 1 (routed + pseudo shared rows when fused): weights W13 once, x once, h written once
    s1_w = active * 2.0 * H * I * bw + (2.0 * H * Is * bw if (Is and m_pseudo) else 0.0)
    s1_bytes = s1_w + T * H * bx + (P + (T * m_pseudo if m_pseudo else 0)) * I * bh
    s1_flops = 4.0 * H * I * P + (4.0 * H * Is * T if m_pseudo else 0.0)
    # stage 2: W2 once, h read once, out written once
    s2_w = active * 1.0 * H * I * bw + (1.0 * H * Is * bw if (Is and m_pseudo) else 0.0)
    s2_bytes = s2_w + (P + (T * m_pseudo if m_pseudo else 0)) * I * bh + T * H * bo
    s2_flops = 2.0 * H * I * P + (2.0 * H * Is * T if m_pseudo else 0.0)
    return flops, byt, (s1_flops, s1_bytes), (s2_flops, s2_bytes), active


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, seconds):
    """The oracle as it stands, on this host's cores, over passes of the same
    workload until ``seconds`` have elapsed: every token of the small
    workloads, a fixed seeded token sample of the large ones (each pass
    routes all T tokens and runs every expert the sample selects, decoding
    those experts' weights from the same bytes the GPU reads)."""
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    lazy = cfg.T * cfg.topk >= cfg.E * 4
    host = workloads.to_host(inp, lazy_weights=lazy)
    n_tok = {"a8w8_large": 4, "mxfp8": 16, "prefill_bf16": 64}.get(cfg.name, cfg.T)
    tokens = np.sort(np.random.default_rng(20261203).choice(cfg.T, size=n_tok, replace=False))
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.moe_layer(host, cfg, tokens=tokens)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    sample = (f"{n} oracle passes over {tokens.size} of the {cfg.T} tokens of {cfg.name} "
              f"(seeded sample; routing of all {cfg.T} tokens in every pass), {el:.1f} s "
              f"on {cpu_model()}")
    return {"value": n * tokens.size / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": sample}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this layer runs on one GPU; --gpus N with N > 1 is not supported "
                                   "(the library has no collectives or sharding)"}))
        sys.exit(2)
    import torch
    import workloads
    import routed_shared_experts_amd as m

    dev = torch.device("cuda:0")
    cfg = workloads.CONFIGS[args.workload]
    if args.router:
        cfg = cfg.replace(router_std=float(cfg.H) ** -0.5)
    inp = workloads.generate(cfg, device=dev)
    wbytes = workloads.bytes_per_weight(cfg.fmt) * 3.0 * cfg.H * (cfg.E * cfg.I + cfg.I_s)
    copies = args.copies or max(1, min(6, int(np.ceil(3 * 256e6 / wbytes))))
    # rotate weight copies so the per-step footprint exceeds the 256 MB Infinity
    # Cache; each copy is a tiled (load-time packed) set of the same weights
    packed_sets = [m.pack_weights(cfg, inp) for _ in range(copies)]
    torch.cuda.synchronize()

    modes = ["pseudo", "aux"] if args.mode == "best" else [args.mode]
    results = {}
    for mode in modes:
        layers = [m.MoeLayer(cfg, inp, shared_mode=mode, packed=pk, block_m=args.block_m) for pk in packed_sets]
        out = layers[0].out
        for L in layers[1:]:
            L.args.out = m._ptr(out)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(N_EVENTS)] for _ in range(args.steps)]
        stream = torch.cuda.current_stream()
        for e in evs:
            for x in e:
                x.record(stream)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            layers[i % copies].forward()
        torch.cuda.synchronize()

        if args.graph:
            graphs = []
            for L in layers:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    L.forward()
                graphs.append(g)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(args.steps):
                graphs[i % copies].replay()
            torch.cuda.synchronize()
            el = time.perf_counter() - t0
            stage = None
        else:
            # live per-kernel timing on every TIMING_EVERY-th step: events
            # between the prologue launches on the main stream, and events
            # stamped with each GEMM kernel's own start and end
            handles = [m.ctypes.cast((m.c_void_p * N_EVENTS)(*[x.cuda_event for x in e]), m.c_void_p) for e in evs]
            timed = [i for i in range(args.steps) if i % TIMING_EVERY == 0]
            t0 = time.perf_counter()
            for i in range(args.steps):
                L = layers[i % copies]
                L.args.timing_events = handles[i] if i % TIMING_EVERY == 0 else None
                L.forward()
            torch.cuda.synchronize()
            el = time.perf_counter() - t0
            for L in layers:
                L.args.timing_events = None
            spans = {"prologue": (0, 1), "sort": (1, 2), "stage1": (3, 4), "stage2": (5, 6)}
            stage = {n: float(np.mean([evs[i][a].elapsed_time(evs[i][b]) for i in timed]))
                     for n, (a, b) in spans.items()}
        results[mode] = (el, stage, layers[0])
        del layers

    best = min(results, key=lambda k: results[k][0])
    el, stage, layer = results[best]
    ms = el / args.steps * 1e3
    # routing result of the timed workload (for the algorithmic byte count)
    ids = torch.empty((cfg.T, cfg.topk), dtype=torch.int32, device=dev)
    w = torch.empty((cfg.T, cfg.topk), dtype=torch.float32, device=dev)
    logits = inp["logits"]
    if logits is None:  # router-GEMM mode: the same logits the layer computed
        logits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=dev)
        m.moe_router_logits(inp["x"], inp["router_w"], logits, x_row_scale=inp.get("x_scale"))
    m.moe_route(logits, ids, w, topk=cfg.topk, bias=inp.get("bias"), n_group=cfg.n_group,
                topk_group=cfg.topk_group, group_score_topk=cfg.group_score_topk,
                score=m.MOE_SCORE_SIGMOID if cfg.score == "sigmoid" else m.MOE_SCORE_SOFTMAX,
                renormalize=cfg.renormalize, routed_scaling_factor=cfg.routed_scaling_factor)
    torch.cuda.synchronize()
    m_pseudo = cfg.n_pseudo if best == "pseudo" else 0
    flops, byt, s1, s2, active = algorithmic(cfg, ids.cpu().numpy(), m_pseudo)
    if args.router:  # the router GEMM: its FLOPs and its weights once
        flops += 2.0 * cfg.T * cfg.E * cfg.H
        byt += cfg.E * cfg.H * (4 if cfg.fmt == "f32" else 2)
    rec = {
        "metric": METRIC,
        "value": cfg.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[cfg.fmt],
        "data": "synthetic (seeded; random-init weights of the workload's shapes)",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "I": cfg.I, "I_s": cfg.I_s,
                   "topk": cfg.topk, "score": cfg.score, "shared_mode": best, "weight_copies": copies,
                   "graph": bool(args.graph), "router_gemm": bool(args.router), "active_experts": active},
        "layer": {"tflops": flops / (ms * 1e-3) / 1e12, "gbps": byt / (ms * 1e-3) / 1e9,
                  "frac_mfma": flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[cfg.fmt],
                  "frac_hbm": byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                  "algorithmic_bytes": byt, "algorithmic_flops": flops},
        "modes_ms": {k: v[0] / args.steps * 1e3 for k, v in results.items()},
    }
    if stage is not None:
        rec["kernels_ms"] = stage
        # the dominant GEMM stage, against HBM or the MFMA peak of its dtype,
        # whichever its arithmetic intensity makes the bound
        st = "stage1" if stage["stage1"] >= stage["stage2"] else "stage2"
        s_flops, s_bytes = s1 if st == "stage1" else s2
        s_ms = stage[st]
        peak_f = MFMA_PEAK_TFLOPS[cfg.fmt]
        mfma_bound = s_flops / s_bytes > peak_f * 1e12 / (HBM_PEAK_GBS * 1e9)
        names = {"stage1": "gemm stage 1 (routed gate/up + SiLU-mul)",
                 "stage2": "gemm stage 2 (down + weighted reduction onto the addend)"}
        if mfma_bound:
            ach, peak, unit = s_flops / (s_ms * 1e-3) / 1e12, peak_f, "TFLOP/s"
        else:
            ach, peak, unit = s_bytes / (s_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
        rec["roofline"] = {"kernel": names[st], "bound": "mfma" if mfma_bound else "hbm",
                           "achieved": ach, "peak": peak, "unit": unit, "frac": ach / peak,
                           "traffic": measured_traffic(cfg.name, st) if best == "pseudo" else None,
                           "bytes_per_launch": s_bytes, "flops_per_launch": s_flops,
                           "timed_steps": len(range(0, args.steps, TIMING_EVERY))}
    if args.copy_calibration > 0:
        n = int(args.copy_calibration * 2**20) // 16 * 16
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_calibration_bytes"] = n
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
