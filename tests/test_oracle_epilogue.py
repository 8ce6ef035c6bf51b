"""Pins of the oracle's epilogue variants: the per-expert biases and the
GELU activation (AITER PR 6106, Technical Details: scales, then bias, then
activation and fused quantisation on the fp32 accumulator).

* the two activations against torch's float64 library routines;
* the stage-2 bias against its closed form: by linearity the layer with b2
  differs from the layer without it by exactly sum_j w_tj b2[e_tj] + gamma_t
  bs2 for every token;
* the stage-1 bias against an extra input column: x' = [x, 1] with W13' =
  [W13, b13] gives x' . W13'^T = x . W13^T + b13, so the layer with b13 equals
  the layer without it on the widened input.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads


def _cfg(fmt, act="silu", **kw):
    base = dict(name=f"epi_{fmt}_{act}", T=40, H=64 if fmt in ("f32", "bf16") else 256, E=6,
                I=32 if fmt in ("f32", "bf16") else 256, I_s=64 if fmt in ("f32", "bf16") else 256, topk=2,
                fmt=fmt, bias13_std=0.05, bias2_std=0.05, activation=act, gated=fmt in ("f32", "bf16"))
    base.update(kw)
    return workloads.LayerConfig(**base)


def test_activations_match_torch():
    g = np.concatenate([np.linspace(-30.0, 30.0, 60001), [0.0, -0.0, 1e-30, -1e-30, 5.5, -5.5]])
    gt = torch.from_numpy(g)
    silu = torch.nn.functional.silu(gt).numpy()
    gelu = torch.nn.functional.gelu(gt, approximate="tanh").numpy()
    np.testing.assert_allclose(oracle.activation(g, "silu"), silu, rtol=1e-13, atol=1e-300)
    # for large negative g both evaluate 1 + tanh(z) by cancellation: compare
    # there to within a few ulp of |g|
    assert (np.abs(oracle.activation(g, "gelu_tanh") - gelu) <= 1e-13 * np.abs(gelu) + 1e-15 * np.abs(g)).all()
    with pytest.raises(ValueError):
        oracle.activation(g, "relu")


@pytest.mark.parametrize("fmt", ["f32", "bf16", "mxfp8", "a8w8", "mxfp4"])
@pytest.mark.parametrize("act", ["silu", "gelu_tanh"])
def test_output_bias_closed_form(fmt, act):
    cfg = _cfg(fmt, act)
    host = workloads.to_host(workloads.generate(cfg))
    r = oracle.moe_layer(host, cfg)
    plain = dict(host, b2=None, bs2=None)
    r0 = oracle.moe_layer(plain, cfg)
    b2 = host["b2"].astype(np.float64)
    expect = np.einsum("tj,tjh->th", r["w"], b2[r["ids"]]) + r["gamma"][:, None] * host["bs2"].astype(np.float64)
    np.testing.assert_allclose(r["y"] - r0["y"], expect, rtol=1e-9, atol=1e-12 * np.abs(r["y"]).max())
    # and the bias does reach the output: removing it changes every token
    assert (np.abs(r["y"] - r0["y"]).max(axis=1) > 1e-3 * np.abs(expect).max()).all()


def _widen(host, cfg, fmt):
    """Inputs with one more input column: x' = [x, 1], W13' = [W13, b13]
    (biases rounded to the weight format first so both sides are exact)."""
    T = cfg.T
    h = dict(host)
    if fmt == "f32":
        x = np.concatenate([host["x"], np.ones((T, 1), np.float32)], axis=1)
        b13 = host["b13"].astype(np.float32)
        bs13 = host["bs13"].astype(np.float32)
    else:
        one = oracle.round_to_bf16_bits(np.ones((T, 1)))
        x = np.concatenate([host["x"], one], axis=1)
        b13_bits = oracle.round_to_bf16_bits(host["b13"].astype(np.float64))
        bs13_bits = oracle.round_to_bf16_bits(host["bs13"].astype(np.float64))
        b13 = oracle.bf16_bits_to_f64(b13_bits).astype(np.float32)
        bs13 = oracle.bf16_bits_to_f64(bs13_bits).astype(np.float32)
    h["x"] = x
    if fmt == "f32":
        h["w13"] = np.concatenate([host["w13"], b13[:, :, None]], axis=2)
        h["ws13"] = np.concatenate([host["ws13"], bs13[:, None]], axis=1)
    else:
        h["w13"] = np.concatenate([host["w13"], oracle.round_to_bf16_bits(b13.astype(np.float64))[:, :, None]], axis=2)
        h["ws13"] = np.concatenate([host["ws13"], oracle.round_to_bf16_bits(bs13.astype(np.float64))[:, None]], axis=1)
    if host.get("gate_w") is not None:
        zero = np.zeros(1, np.float32) if fmt == "f32" else oracle.round_to_bf16_bits(np.zeros(1))
        h["gate_w"] = np.concatenate([host["gate_w"], zero])
    h["b13"], h["bs13"] = None, None
    with_bias = dict(host, b13=b13, bs13=bs13)
    return with_bias, h


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
@pytest.mark.parametrize("act", ["silu", "gelu_tanh"])
def test_stage1_bias_is_an_extra_input_column(fmt, act):
    cfg = _cfg(fmt, act, bias13_std=0.3)
    host = workloads.to_host(workloads.generate(cfg))
    with_bias, wide = _widen(host, cfg, fmt)
    y = oracle.moe_layer(with_bias, cfg)["y"]
    yw = oracle.moe_layer(wide, cfg)["y"]   # (the output width stays H)
    # equal up to the float64 order of one extra product, which can move h
    # across a rounding boundary of its own format (fp32 or bf16) now and then
    tol = (2.0 ** -20 if fmt == "f32" else 2.0 ** -10) * np.abs(y).max()
    assert np.abs(y - yw).max() <= tol
    assert np.mean(np.isclose(y, yw, rtol=1e-9, atol=1e-12)) > 0.9
    # the comparison has teeth: the layer without the stage-1 bias is far off
    wrong = oracle.moe_layer(dict(host, b13=None, bs13=None), cfg)["y"]
    assert np.abs(wrong - y).max() > 10 * tol


@pytest.mark.parametrize("fmt", ["f32", "bf16", "mxfp8", "a8w8"])
def test_router_logits_brute_force(fmt):
    """oracle.router_logits against an explicit sum over k of x_tk w_ek from
    the decoded inputs, on a tiny case (a8w8: the token's scale times the
    codes; MX formats: the bf16 input before its quantisation)."""
    cfg = workloads.LayerConfig(name=f"rl_{fmt}", T=3, H=64 if fmt != "a8w8" else 64, E=5, I=32, I_s=0, topk=2,
                                fmt=fmt, gated=False, router_std=0.1)
    host = workloads.to_host(workloads.generate(cfg))
    got = oracle.router_logits(host, fmt)
    if fmt == "f32":
        x = host["x"].astype(np.float64)
        w = host["router_w"].astype(np.float64)
    else:
        w = oracle.bf16_bits_to_f64(host["router_w"])
        if fmt == "a8w8":
            x = oracle.e4m3_decode(host["x"]) * host["x_scale"].astype(np.float64)[:, None]
        else:
            x = oracle.bf16_bits_to_f64(host["x"])
    for t in range(cfg.T):
        for e in range(cfg.E):
            s = 0.0
            for k in range(cfg.H):
                s += x[t, k] * w[e, k]
            assert abs(got[t, e] - s) <= 1e-12 * (np.abs(x[t]) @ np.abs(w[e]))
    # the layer routes on these logits rounded to fp32 when it has no logits input
    assert host["logits"] is None
    ids, _ = oracle.route(got.astype(np.float32), topk=cfg.topk)
    r = oracle.moe_layer(host, cfg)
    assert np.array_equal(r["ids"], ids)
