"""Independent pins of the oracle's fp8 expert chain and of the biased sigmoid
routing weights.

The reference below is written here, from the format definitions, with torch
float64 arithmetic and torch's own float8_e4m3fn / bfloat16 casts; it calls
nothing in ``oracle``.  One routed expert (E = 1, k = 1, no shared expert) in
the MXFP8 and a8w8 formats:

* scales on the fp32 accumulator before the activation, MX scales per
  32-element K block (AITER PR 6106, Technical Details);
* h rounded to bf16 before any fp8 quantisation, then MX-32 (OCP MX v1.0:
  X = floor(log2 amax) - 8, codes = e4m3(v * 2^-X) saturated) or per row
  (s = amax / 448, codes = e4m3(v * (448 / amax)));
* o = (h_q . W2^T) * s_h * s2.

Planted mistakes in the oracle (dropping the bf16 rounding of h, the h
quantisation or the row scale) must make the comparison fail: the last tests
check exactly that by patching the oracle on the CPU.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import layer as L

F8 = torch.float8_e4m3fn


def _cfg(fmt):
    return workloads.LayerConfig(name=f"fp8chain_{fmt}", T=24, H=256, E=1, I=128, I_s=0, topk=1,
                                 fmt=fmt, gated=False, score="softmax", logits="iid")


def _e4m3_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(F8).double()


def _to_e4m3(v32):
    """float32 tensor -> e4m3 values (float64): torch's RNE cast after clamping
    to the largest finite magnitude (the cast itself overflows to NaN)."""
    return v32.clamp(-448.0, 448.0).to(F8).double()


def _bf16(h64):
    """Round float64 to bf16 (as float64).  torch rounds through float32;
    that double rounding can differ from one rounding only when the float32
    value is a bf16 tie that the float64 value was not, which the caller
    rules out for its inputs."""
    h32 = h64.float()
    bits = h32.view(torch.int32)
    tie = ((bits & 0xFFFF) == 0x8000) & (h32.double() != h64)
    assert not bool(tie.any()), "double-rounding case in the test input; pick another seed"
    return h32.to(torch.bfloat16).double()


def _mx_quant(v32):
    """MX-32 along the last axis -> dequantised float64 values."""
    n, k = v32.shape
    b = v32.reshape(n, k // 32, 32)
    amax = b.abs().amax(dim=-1)
    _, e = torch.frexp(amax)                       # amax = m 2^e, m in [0.5, 1)
    X = torch.where(amax > 0, e - 1 - 8, torch.full_like(e, -127)).clamp(-127, 127)
    scaled = torch.ldexp(b, (-X)[..., None].float())
    q = _to_e4m3(scaled.float())
    return (q * torch.ldexp(torch.ones_like(q), X[..., None].double())).reshape(n, k)


def _row_quant(v32):
    """Per-row e4m3 -> (codes as float64 values, row scale float64)."""
    amax = v32.abs().amax(dim=-1)
    nz = amax > 0
    safe = torch.where(nz, amax, torch.ones_like(amax))
    inv = torch.tensor(448.0, dtype=torch.float32) / safe        # float32 division
    s = safe / torch.tensor(448.0, dtype=torch.float32)
    q = _to_e4m3((v32 * inv[:, None]).float())
    q = torch.where(nz[:, None], q, torch.zeros_like(q))
    return q, torch.where(nz, s, torch.ones_like(s)).double()


def _e2m1_table():
    """The 16 e2m1 values from the OCP MX specification's table (golden file)."""
    import os
    vals = []
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "e2m1_values.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            vals.append(float(line.split()[1]))
    return torch.tensor(vals, dtype=torch.float64)


def torch_expert(inp, fmt):
    """One routed expert in fp8 / MXFP4, from the definitions (no oracle code)."""
    if fmt in ("mxfp8", "mxfp4"):
        x32 = torch.from_numpy(inp["x"].astype(np.uint32) << 16).view(torch.float32)
        x = _mx_quant(x32)
        sx = torch.ones(x.shape[0], dtype=torch.float64)
        def wdec(codes, sc):
            if fmt == "mxfp8":
                v = _e4m3_values(codes)
            else:  # two e2m1 codes per byte, the even element in the low nibble
                b = torch.from_numpy(np.ascontiguousarray(codes)).long()
                v = torch.stack([_e2m1_table()[b & 15], _e2m1_table()[b >> 4]], dim=-1).reshape(b.shape[0], -1)
            ex = torch.from_numpy(sc.astype(np.int64) - 127).double()
            return v * torch.ldexp(torch.ones_like(v), ex.repeat_interleave(32, dim=-1))
        W13 = wdec(inp["w13"][0], inp["w13_scale"][0])
        W2 = wdec(inp["w2"][0], inp["w2_scale"][0])
        s13 = s2 = 1.0
    else:
        x = _e4m3_values(inp["x"])
        sx = torch.from_numpy(inp["x_scale"]).double()
        W13 = _e4m3_values(inp["w13"][0])
        W2 = _e4m3_values(inp["w2"][0])
        s13 = float(inp["w13_scale"][0])
        s2 = float(inp["w2_scale"][0])
    I = W2.shape[1]
    a = (x @ W13.T) * sx[:, None] * s13
    h = torch.nn.functional.silu(a[:, :I]) * a[:, I:]
    hb = _bf16(h)
    if fmt in ("mxfp8", "mxfp4"):
        hq, sh = _mx_quant(hb.float()), torch.ones(h.shape[0], dtype=torch.float64)
    else:
        hq, sh = _row_quant(hb.float())
    o = (hq @ W2.T) * sh[:, None] * s2
    return o.numpy(), hq.numpy()


def _compare(fmt):
    cfg = _cfg(fmt)
    inp = workloads.to_host(workloads.generate(cfg))
    y = oracle.moe_layer(inp, cfg)["y"]
    ref, _ = torch_expert(inp, fmt)
    rms = np.sqrt((ref ** 2).mean())
    return np.abs(y - ref).max() / rms


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "a8w8"])
def test_fp8_expert_chain_matches_independent_torch_reference(fmt):
    # the two differ only in the float64 summation order of the products
    assert _compare(fmt) <= 1e-12


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "a8w8"])
def test_fp8_h_codes_match_independent_torch_reference(fmt):
    cfg = _cfg(fmt)
    inp = workloads.to_host(workloads.generate(cfg))
    xh, sx = L.decode_activations(inp, fmt)
    W13, W2, s13, s2 = L.expert_weights(inp, fmt, 0)
    _, inter = L.expert_mlp(xh, sx, W13, W2, s13, s2, fmt, intermediates=True)
    _, hq = torch_expert(inp, fmt)
    assert np.array_equal(inter["h_tilde"], hq)


def _planted(monkeypatch, fmt, mistake):
    real = L.quantize_h

    def no_bf16(h, f):
        if f in ("mxfp8", "mxfp4"):
            sc, q = oracle.mx_quantize(h.astype(np.float32))
            return oracle.mx_dequantize(sc, q), np.ones(h.shape[0])
        s, q = oracle.row_quantize_e4m3(h.astype(np.float32))
        return oracle.e4m3_decode(q), s.astype(np.float64)

    def no_quant(h, f):
        return oracle.bf16_bits_to_f64(oracle.round_to_bf16_bits(h)), np.ones(h.shape[0])

    def no_row_scale(h, f):
        ht, _ = real(h, f)
        return ht, np.ones(h.shape[0])

    monkeypatch.setattr(L, "quantize_h", {"no_bf16": no_bf16, "no_quant": no_quant,
                                          "no_row_scale": no_row_scale}[mistake])


@pytest.mark.parametrize("fmt,mistake", [("mxfp8", "no_bf16"), ("mxfp8", "no_quant"), ("mxfp4", "no_bf16"),
                                         ("mxfp4", "no_quant"), ("a8w8", "no_bf16"),
                                         ("a8w8", "no_quant"), ("a8w8", "no_row_scale")])
def test_planted_oracle_mistakes_are_caught(monkeypatch, fmt, mistake):
    _planted(monkeypatch, fmt, mistake)
    assert _compare(fmt) > 1e-6


def test_biased_sigmoid_weights_closed_form():
    """Selection on sigmoid(logit) + bias, weights from the unbiased sigmoid,
    renormalised, times the routed scale (vLLM PR 65207, Purpose, commit 1:
    biased grouped top-k with the scale folded in).  The bias lifts experts 5
    and 7 over higher-logit ones by wide margins, so the selection is plain,
    and the weights are sigmoid(l_j) / sum_sel sigmoid(l) * s in closed form."""
    lg = np.array([[2.0, 1.5, 1.0, 0.0, -1.0, -1.5, -2.0, -3.0]], np.float32)
    bias = np.array([0, 0, 0, 0, 0, 1.0, 0, 2.0], np.float32)
    sig = [1.0 / (1.0 + math.exp(-float(v))) for v in lg[0]]
    ids, w = oracle.route(lg, topk=2, score="sigmoid", bias=bias, routed_scaling_factor=2.5)
    assert ids.tolist() == [[7, 5]]
    tot = sig[7] + sig[5]
    assert np.allclose(w[0], [sig[7] / tot * 2.5, sig[5] / tot * 2.5], rtol=1e-15, atol=0)
    # groups of two (top-2 sums 1.699, 1.231, 1.451, 2.166): groups 3 and 0 kept
    ids, w = oracle.route(lg, topk=2, score="sigmoid", bias=bias, n_group=4, topk_group=2,
                          routed_scaling_factor=2.5)
    assert ids.tolist() == [[7, 0]]
    tot = sig[7] + sig[0]
    assert np.allclose(w[0], [sig[7] / tot * 2.5, sig[0] / tot * 2.5], rtol=1e-15, atol=0)
    # without renormalisation the weights are the plain sigmoids times the scale
    ids, w = oracle.route(lg, topk=2, score="sigmoid", bias=bias, renormalize=False, routed_scaling_factor=2.5)
    assert np.allclose(w[0], [sig[7] * 2.5, sig[5] * 2.5], rtol=1e-15, atol=0)
