"""Seeded synthetic inputs for the MoE layer: the five workload shapes.

This module only draws random numbers and packs them into the layer's input
formats; it holds none of the layer's arithmetic.  Both the GPU path (through
``bench.py`` and the tests) and the CPU oracle consume the exact bytes it
produces.  Quantised inputs are drawn directly in their quantised form (random
e4m3 codes from torch's float8 cast of scaled normal draws, random scale
exponents), so no quantiser of the layer lives here.

Workloads (the tiny one is small enough for the oracle to finish in seconds):

* tiny_f32      T=8,    H=64,   E=4,   I=32,   k=2, shared I_s=64,   softmax, gated
* decode_bf16   T=32,   H=2048, E=64,  I=512,  k=8, shared I_s=512,  softmax, gated
* prefill_bf16  T=4096, H=2048, E=64,  I=512,  k=8, shared I_s=2048, softmax, gated,
                Zipf(1.1) expert load
* mxfp8         T=512,  H=4096, E=128, I=1536, k=8, shared I_s=1536, sigmoid + bias,
                8 groups keep 4, routed scaling 2.5, MX-32 e4m3 weights, ungated
* a8w8_large    T=8192, H=7168, E=256, I=2048, k=8, shared I_s=2048, sigmoid,
                8 groups keep 4, e4m3 activations (fp32 per token) and weights
                (fp32 per expert), Zipf(1.2) expert load, ungated
* mxfp4, mxfp4_decode  the mxfp8 shape (T=512; T=32) with MXFP4 weights (e2m1
                codes drawn at random, two per byte, e8m0 scale per 32)

Zipf load uses the Gumbel-top-k construction (Kool, van Hoof & Welling 2019):
logits[t, e] = ln p_{pi(e)} + G_te with G standard Gumbel, p_r proportional to
r^-s and pi a seeded permutation, so that top-k by logit draws k experts without
replacement in proportion to p.
"""

import dataclasses
import hashlib

import numpy as np
import torch

BASE_SEED = 20261203


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    H: int
    E: int
    I: int
    I_s: int
    topk: int
    score: str = "softmax"
    n_group: int = 1
    topk_group: int = 1
    group_score_topk: int = 2
    renormalize: bool = True
    routed_scaling_factor: float = 1.0
    fmt: str = "bf16"            # 'f32' | 'bf16' | 'mxfp8' | 'mxfp4' | 'a8w8'
    gated: bool = True
    bias_std: float = 0.0
    logits: str = "iid"          # 'linear' | 'iid' | 'zipf'
    zipf_s: float = 0.0
    bias13_std: float = 0.0      # std of the per-expert fp32 stage-1 biases b13, bs13 (0: none)
    bias2_std: float = 0.0       # std of the per-expert fp32 stage-2 biases b2, bs2 (0: none)
    activation: str = "silu"     # 'silu' | 'gelu_tanh'
    router_std: float = 0.0      # > 0: router projection [E, H] ~ N(0, std^2) in x's precision, and the
                                 # layer computes its own logits (the logits input is then None)

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)

    @property
    def n_pseudo(self):
        return -(-self.I_s // self.I) if self.I_s > 0 else 0


CONFIGS = {
    "tiny_f32": LayerConfig("tiny_f32", T=8, H=64, E=4, I=32, I_s=64, topk=2, fmt="f32",
                            logits="linear"),
    "decode_bf16": LayerConfig("decode_bf16", T=32, H=2048, E=64, I=512, I_s=512, topk=8,
                               fmt="bf16", logits="iid"),
    "prefill_bf16": LayerConfig("prefill_bf16", T=4096, H=2048, E=64, I=512, I_s=2048, topk=8,
                                fmt="bf16", logits="zipf", zipf_s=1.1),
    "mxfp8": LayerConfig("mxfp8", T=512, H=4096, E=128, I=1536, I_s=1536, topk=8,
                         score="sigmoid", n_group=8, topk_group=4, routed_scaling_factor=2.5,
                         fmt="mxfp8", gated=False, bias_std=0.1, logits="iid"),
    "a8w8_large": LayerConfig("a8w8_large", T=8192, H=7168, E=256, I=2048, I_s=2048, topk=8,
                              score="sigmoid", n_group=8, topk_group=4, fmt="a8w8",
                              gated=False, logits="zipf", zipf_s=1.2),
}
CONFIG_ORDER = ["tiny_f32", "decode_bf16", "prefill_bf16", "mxfp8", "a8w8_large"]

# MXFP4 expert weights with MX-fp8 activations (the format the pages deploy,
# vLLM PR 65207, Purpose, commit 3): the MXFP8 workload's shape with e2m1
# weights, and a decode batch of it
CONFIGS["mxfp4"] = CONFIGS["mxfp8"].replace(name="mxfp4", fmt="mxfp4")
CONFIGS["mxfp4_decode"] = CONFIGS["mxfp8"].replace(name="mxfp4_decode", fmt="mxfp4", T=32)


def _seed(*key):
    h = hashlib.sha256(repr((BASE_SEED,) + tuple(key)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *key):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*key))
    return g


def _randn(shape, device, *key):
    return torch.randn(shape, generator=_gen(device, *key), device=device, dtype=torch.float32)


def _e4m3(t):
    """Draws already scaled into the e4m3 range -> e4m3 codes (uint8)."""
    return t.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def _weight_family(cfg, device, tag, n_mats, rows, cols, fmt):
    """n_mats matrices [rows, cols]; returns (values, scales) in the layer format."""
    shape = (n_mats, rows, cols)
    if fmt == "f32":
        out = torch.empty(shape, dtype=torch.float32, device=device)
    elif fmt == "bf16":
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    elif fmt == "mxfp4":
        out = torch.empty((n_mats, rows, cols // 2), dtype=torch.uint8, device=device)
    else:
        out = torch.empty(shape, dtype=torch.uint8, device=device)
    scales = None
    if fmt in ("mxfp8", "mxfp4"):
        scales = torch.empty((n_mats, rows, cols // 32), dtype=torch.uint8, device=device)
    elif fmt == "a8w8":
        scales = torch.empty((n_mats,), dtype=torch.float32, device=device)
    for e in range(n_mats):
        r = _randn((rows, cols), device, cfg.name, tag, e) if fmt != "mxfp4" else None
        if fmt == "f32":
            out[e] = r.mul_(0.02)
        elif fmt == "bf16":
            out[e] = r.mul_(0.02).to(torch.bfloat16)
        elif fmt == "mxfp8":
            # codes ~ N(0, 16^2) with block exponents 2^-11 .. 2^-9: values ~ N(0, ~0.02^2)
            out[e] = _e4m3(r.mul_(16.0))
            g = _gen(device, cfg.name, tag + "_scale", e)
            scales[e] = torch.randint(116, 119, (rows, cols // 32), generator=g, device=device,
                                      dtype=torch.int32).to(torch.uint8)
        elif fmt == "mxfp4":
            # e2m1 codes 0..15 drawn from a fixed bell-shaped distribution over
            # the magnitudes (0, 0.5, 1, 1.5, 2, 3, 4, 6) with a random sign, two
            # per byte, and block exponents 2^-8 .. 2^-6: values of order 0.02
            g = _gen(device, cfg.name, tag + "_codes", e)
            mag = torch.multinomial(_E2M1_MAG_P.to(device), rows * cols, replacement=True, generator=g)
            sign = torch.randint(0, 2, (rows * cols,), generator=g, device=device)
            codes = (mag + 8 * sign).to(torch.uint8).view(rows, cols)
            out[e] = codes[:, 0::2] | (codes[:, 1::2] << 4)
            g = _gen(device, cfg.name, tag + "_scale", e)
            scales[e] = torch.randint(119, 122, (rows, cols // 32), generator=g, device=device,
                                      dtype=torch.int32).to(torch.uint8)
        elif fmt == "a8w8":
            out[e] = _e4m3(r.mul_(64.0))
            g = _gen(device, cfg.name, tag + "_scale", e)
            u = torch.rand((1,), generator=g, device=device, dtype=torch.float32)
            scales[e] = (0.02 / 64.0) * (0.9 + 0.2 * u[0])
    return out, scales


# probabilities of the e2m1 magnitude codes 0..7 (values 0, 0.5, 1, 1.5, 2,
# 3, 4, 6) for random MXFP4 weights: a bell over the grid
_E2M1_MAG_P = torch.tensor([0.10, 0.20, 0.20, 0.16, 0.14, 0.11, 0.06, 0.03], dtype=torch.float64)


def _zipf_logits(cfg, device):
    g = _gen("cpu", cfg.name, "zipf_perm")
    perm = torch.randperm(cfg.E, generator=g)
    ranks = torch.arange(1, cfg.E + 1, dtype=torch.float64)
    p = ranks.pow(-cfg.zipf_s)
    p = p / p.sum()
    lnp = torch.log(p)[perm].to(device)
    u = torch.rand((cfg.T, cfg.E), generator=_gen(device, cfg.name, "gumbel"), device=device,
                   dtype=torch.float64)
    u = u.clamp_(1e-300, 1.0 - 1e-16)
    gumbel = -torch.log(-torch.log(u))
    return (lnp[None, :] + gumbel).to(torch.float32)


def generate(cfg, device="cpu"):
    """All layer inputs as torch tensors on ``device`` (dict, oracle key names)."""
    T, H, E, I, I_s = cfg.T, cfg.H, cfg.E, cfg.I, cfg.I_s
    inp = {}
    # activations
    xr = _randn((T, H), device, cfg.name, "x")
    if cfg.fmt == "f32":
        inp["x"] = xr
    elif cfg.fmt in ("bf16", "mxfp8", "mxfp4"):
        inp["x"] = xr.to(torch.bfloat16)
    else:  # a8w8: e4m3 codes ~ N(0, 100^2) and a per-token fp32 scale near 1/100
        inp["x"] = _e4m3(xr.mul_(100.0))
        u = torch.rand((T,), generator=_gen(device, cfg.name, "x_scale"), device=device)
        inp["x_scale"] = (0.5 + u) / 100.0
    # router logits (an input of the layer)
    if cfg.logits == "linear":
        wr = torch.randn((E, H), generator=_gen("cpu", cfg.name, "router"), dtype=torch.float64) * 0.1
        inp["logits"] = (xr.detach().cpu().double() @ wr.T).to(torch.float32).to(device)
    elif cfg.logits == "iid":
        inp["logits"] = _randn((T, E), device, cfg.name, "logits")
    else:
        inp["logits"] = _zipf_logits(cfg, device)
    inp["router_w"] = None
    if cfg.router_std > 0:
        wr = _randn((E, H), device, cfg.name, "router_w") * cfg.router_std
        inp["router_w"] = wr if cfg.fmt == "f32" else wr.to(torch.bfloat16)
        inp["logits"] = None
    inp["bias"] = (_randn((E,), device, cfg.name, "bias") * cfg.bias_std) if cfg.bias_std > 0 else None
    if cfg.gated:
        gw = _randn((H,), device, cfg.name, "gate") * 0.02
        inp["gate_w"] = gw if cfg.fmt == "f32" else gw.to(torch.bfloat16)
    else:
        inp["gate_w"] = None
    # routed experts: W13 [E, 2I, H] (gate rows then up rows), W2 [E, H, I]
    inp["w13"], inp["w13_scale"] = _weight_family(cfg, device, "w13", E, 2 * I, H, cfg.fmt)
    inp["w2"], inp["w2_scale"] = _weight_family(cfg, device, "w2", E, H, I, cfg.fmt)
    # shared expert: Ws13 [2I_s, H], Ws2 [H, I_s]
    if I_s > 0:
        ws13, s13 = _weight_family(cfg, device, "ws13", 1, 2 * I_s, H, cfg.fmt)
        ws2, s2 = _weight_family(cfg, device, "ws2", 1, H, I_s, cfg.fmt)
        inp["ws13"], inp["ws2"] = ws13[0], ws2[0]
        mx = cfg.fmt in ("mxfp8", "mxfp4")
        inp["ws13_scale"] = None if s13 is None else (s13[0] if mx else s13)
        inp["ws2_scale"] = None if s2 is None else (s2[0] if mx else s2)
    else:
        inp["ws13"] = inp["ws2"] = inp["ws13_scale"] = inp["ws2_scale"] = None
    # per-expert biases (fp32): b13 [E, 2I], b2 [E, H]; shared bs13 [2 I_s], bs2 [H]
    for k in ("b13", "b2", "bs13", "bs2"):
        inp[k] = None
    if cfg.bias13_std > 0:
        inp["b13"] = _randn((E, 2 * I), device, cfg.name, "b13") * cfg.bias13_std
        if I_s > 0:
            inp["bs13"] = _randn((2 * I_s,), device, cfg.name, "bs13") * cfg.bias13_std
    if cfg.bias2_std > 0:
        inp["b2"] = _randn((E, H), device, cfg.name, "b2") * cfg.bias2_std
        if I_s > 0:
            inp["bs2"] = _randn((H,), device, cfg.name, "bs2") * cfg.bias2_std
    return inp


def _np(t):
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class LazyRows:
    """Index-on-demand host view of a (possibly device) tensor's first axis."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, i):
        return _np(self.t[i])

    def __len__(self):
        return self.shape[0]


def to_host(inp, lazy_weights=False):
    """Host (numpy) copy of the inputs in the oracle's encoding: bf16 as uint16
    bit patterns, e4m3 as uint8 codes.  With ``lazy_weights`` the routed expert
    tensors are copied one expert at a time when the oracle asks for them."""
    out = {}
    for k, v in inp.items():
        if v is None:
            out[k] = None
        elif lazy_weights and k in ("w13", "w2", "w13_scale", "w2_scale"):
            out[k] = LazyRows(v)
        else:
            out[k] = _np(v)
    return out


def realised_load(ids, E):
    """Per-expert pair counts (min, median, max, active) of a routing result."""
    c = np.bincount(np.asarray(ids).reshape(-1), minlength=E)[:E]
    return {"min": int(c.min()), "median": float(np.median(c)), "max": int(c.max()),
            "active": int((c > 0).sum())}


def zipf_expected_share(E, s):
    p = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    return p / p.sum()


def bytes_per_weight(fmt):
    return {"f32": 4.0, "bf16": 2.0, "mxfp8": 1.0 + 1.0 / 32.0, "mxfp4": 0.5 + 1.0 / 32.0, "a8w8": 1.0}[fmt]

