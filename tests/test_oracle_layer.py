"""Pins of the oracle's layer: torch float64 library routines for a single
expert and for the gated shared expert, dense brute force with the unselected
experts' weights zeroed, and the shared-only / scale-folding identities."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import layer as L


def _small(fmt="f32", **kw):
    base = dict(name="pin", T=12, H=64, E=6, I=32, I_s=64, topk=2, fmt=fmt, logits="iid")
    if fmt in ("mxfp8", "mxfp4", "a8w8"):
        base.update(H=128, I=128, I_s=128, gated=False, score="sigmoid", n_group=2, topk_group=1)
    base.update(kw)
    return workloads.LayerConfig(**base)


def _inputs(cfg):
    return workloads.to_host(workloads.generate(cfg))


def _torch_expert(x, w13, w2, I, hround):
    xt, a = torch.from_numpy(x), torch.from_numpy(w13)
    g = xt @ a[:I].T
    u = xt @ a[I:].T
    h = torch.nn.functional.silu(g) * u
    h = hround(h)
    return (h @ torch.from_numpy(w2).T).numpy()


def test_single_expert_matches_torch_f32():
    cfg = _small("f32", E=1, topk=1, I_s=0)
    inp = _inputs(cfg)
    y = oracle.moe_layer(inp, cfg)["y"]
    x = inp["x"].astype(np.float64)
    ref = _torch_expert(x, inp["w13"][0].astype(np.float64), inp["w2"][0].astype(np.float64), cfg.I,
                        lambda h: h.float().double())
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_single_expert_matches_torch_bf16():
    cfg = _small("bf16", E=1, topk=1, I_s=0)
    inp = _inputs(cfg)
    y = oracle.moe_layer(inp, cfg)["y"]
    dec = oracle.bf16_bits_to_f64
    ref = _torch_expert(dec(inp["x"]), dec(inp["w13"][0]), dec(inp["w2"][0]), cfg.I,
                        lambda h: h.to(torch.bfloat16).double())
    # torch rounds fp64 -> bf16 via fp32 (double rounding) on rare ties; allow that
    assert np.allclose(y, ref, rtol=1e-3, atol=1e-6)


def test_shared_expert_and_gate_match_torch():
    cfg = _small("f32", routed_scaling_factor=0.0)  # routed weights all zero -> y = gamma * S(x)
    inp = _inputs(cfg)
    y = oracle.moe_layer(inp, cfg)["y"]
    x = torch.from_numpy(inp["x"].astype(np.float64))
    gamma = torch.sigmoid(x @ torch.from_numpy(inp["gate_w"].astype(np.float64))).numpy()
    s = _torch_expert(x.numpy(), inp["ws13"].astype(np.float64), inp["ws2"].astype(np.float64), cfg.I_s,
                      lambda h: h.float().double())
    assert np.allclose(y, gamma[:, None] * s, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("fmt", ["f32", "bf16", "mxfp8", "mxfp4", "a8w8"])
def test_layer_equals_dense_brute_force(fmt):
    cfg = _small(fmt)
    inp = _inputs(cfg)
    r = oracle.moe_layer(inp, cfg)
    xh, sx = L.decode_activations(inp, fmt)
    dense = np.zeros((cfg.T, cfg.H))
    for e in range(cfg.E):          # every expert on every token
        W13, W2, s13, s2 = L.expert_weights(inp, fmt, e)
        o = L.expert_mlp(xh, sx, W13, W2, s13, s2, fmt)
        wfull = np.zeros(cfg.T)
        for t in range(cfg.T):
            j = np.nonzero(r["ids"][t] == e)[0]
            wfull[t] = r["w"][t, j[0]] if j.size else 0.0
        dense += wfull[:, None] * o
    Ws13, Ws2, s13, s2 = L.shared_weights(inp, fmt)
    dense += r["gamma"][:, None] * L.expert_mlp(xh, sx, Ws13, Ws2, s13, s2, fmt)
    rms = np.sqrt((dense ** 2).mean())
    assert np.abs(r["y"] - dense).max() <= 1e-12 * rms


def test_shared_only_is_exact():
    cfg = _small("bf16", routed_scaling_factor=0.0)
    inp = _inputs(cfg)
    r = oracle.moe_layer(inp, cfg)
    xh, sx = L.decode_activations(inp, "bf16")
    Ws13, Ws2, s13, s2 = L.shared_weights(inp, "bf16")
    s = L.expert_mlp(xh, sx, Ws13, Ws2, s13, s2, "bf16")
    assert np.array_equal(r["y"], r["gamma"][:, None] * s)


def test_routed_scale_fold_identity():
    cfg1 = _small("bf16", I_s=0)
    inp = _inputs(cfg1)
    y1 = oracle.moe_layer(inp, cfg1)["y"]
    y2 = oracle.moe_layer(inp, cfg1.replace(routed_scaling_factor=2.0))["y"]
    assert np.array_equal(y2, 2.0 * y1)  # power-of-two scale: bit-exact
    y25 = oracle.moe_layer(inp, cfg1.replace(routed_scaling_factor=2.5))["y"]
    assert np.allclose(y25, 2.5 * y1, rtol=1e-12, atol=0)


def test_routed_weights_sum_to_scale():
    cfg = _small("bf16", routed_scaling_factor=2.5)
    r = oracle.moe_layer(_inputs(cfg), cfg)
    assert np.all(np.abs(r["w"].sum(1) - 2.5) <= cfg.topk * 2.0 ** -50 * 2.5)


def test_a8w8_scales_on_accumulator_equal_dequantise_first():
    """The oracle's expert applies per-token and per-expert scales to the
    accumulator (AITER PR 6106, Technical Details); with power-of-two scales
    that equals dequantising the operands first, bit for bit, through the
    same function."""
    cfg = _small("a8w8", I_s=0)
    inp = _inputs(cfg)
    sx = np.exp2(np.round(np.log2(inp["x_scale"]))).astype(np.float64)
    xh, _ = L.decode_activations(inp, "a8w8")
    W13, W2, _, _ = L.expert_weights(inp, "a8w8", 0)
    s13, s2 = 2.0 ** -11, 2.0 ** -9
    o_acc = L.expert_mlp(xh, sx, W13, W2, s13, s2, "a8w8")
    o_deq = L.expert_mlp(xh * sx[:, None], np.ones(cfg.T), W13 * s13, W2 * s2, 1.0, 1.0, "a8w8")
    assert np.array_equal(o_acc, o_deq)


def test_pseudo_split_of_shared_expert_is_exact_by_linearity():
    """The shared expert split into ceil(I_s/I) column chunks (the pseudo-expert
    reading of the fused heterogeneous layer) sums to the whole expert."""
    cfg = _small("f32", I=32, I_s=48)
    inp = _inputs(cfg)
    xh, sx = L.decode_activations(inp, "f32")
    Ws13, Ws2, _, _ = L.shared_weights(inp, "f32")
    whole = L.expert_mlp(xh, sx, Ws13, Ws2, 1.0, 1.0, "f32")
    parts = np.zeros_like(whole)
    for c0 in range(0, cfg.I_s, cfg.I):
        c1 = min(c0 + cfg.I, cfg.I_s)
        w13 = np.concatenate([Ws13[c0:c1], Ws13[cfg.I_s + c0:cfg.I_s + c1]])
        parts += L.expert_mlp(xh, sx, w13, Ws2[:, c0:c1], 1.0, 1.0, "f32")
    assert np.allclose(parts, whole, rtol=1e-12, atol=1e-15)


def test_tiny_workload_oracle_runs():
    cfg = workloads.CONFIGS["tiny_f32"]
    r = oracle.moe_layer(_inputs(cfg), cfg)
    assert r["y"].shape == (8, 64) and np.isfinite(r["y"]).all()
