"""The whole MoE layer forward, as a plain per-expert loop in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

For every token t (vLLM PR 65207, Purpose: routed output plus shared-expert
output, with the routed scaling folded into the top-k weights):

    y_t = sum_j w_tj * E_{e_tj}(x_t) + gamma_t * S(x_t)

    E(x) = W2 . Q_h( act(x . Wg^T + bg) * (x . Wu^T + bu) ) + b2
                                                      (gated expert; act = SiLU
                                                       by default)
    gamma_t = sigmoid(x_t . g)                        (vLLM PR 56789, Summary:
                                                       the shared-expert gate is
                                                       sigmoid of a Linear(H, 1))

Weight layout (reading): W13[e] is [2I, H] with the gate rows first and the up
rows second; W2[e] is [H, I]; products are x . W^T.

Quantisation points (AITER PR 6106, Technical Details: per-token activation
scales and per-expert weight scales multiply the fp32 accumulator before the
activation and the fused quantisation; MX GEMMs use 32-element K blocks):

* fmt 'f32':   x, W fp32; the stage-1 output h is rounded to fp32.
* fmt 'bf16':  x, W bf16; h rounded to bf16.
* fmt 'mxfp8': x given in bf16 and quantised to MX-32 e4m3 inside the layer;
               W in MX-32 e4m3; h rounded to bf16 then MX-32 quantised.
* fmt 'a8w8':  x e4m3 with an fp32 scale per token; W e4m3 with an fp32 scale
               per expert (one for W13, one for W2); h rounded to bf16 then
               quantised per row to e4m3 with an fp32 row scale.
* fmt 'mxfp4': as 'mxfp8' (x and h MX-32 e4m3) with MXFP4 weights: e2m1
               elements, an e8m0 scale per 32 K elements.

Expert biases and the activation (AITER PR 6106, Technical Details: the
scales act on the fp32 accumulator before the bias, the activation and the
fused quantisation): the optional fp32 biases b13 = (bg, bu) [2I] are added to
the scaled stage-1 accumulator, b2 [H] to the scaled stage-2 output of the
expert, before its routing weight (or the shared gate) multiplies it -- the
reading of a bias as part of each projection.  act is SiLU, g * sigmoid(g),
or the tanh form of GELU, g/2 * (1 + tanh(sqrt(2/pi) * (g + 0.044715 g^3)))
(the pages name no particular alternative; GELU-gated experts are the common
one).

Every dot product is float64 over the exactly decoded operands, so the only
roundings are the quantisation points themselves.  The shared expert is
evaluated whole (intermediate width I_s), never split.
"""

import numpy as np

from .codecs import (bf16_bits_to_f64, round_to_bf16_bits, e4m3_decode,
                     mx_quantize, mx_dequantize, mx4_dequantize, row_quantize_e4m3)
from .routing import route


def _decode_plain(a, fmt):
    if fmt == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if fmt in ("bf16", "mxfp8"):
        return bf16_bits_to_f64(a)
    raise ValueError(fmt)


def decode_activations(inp, fmt):
    """Layer input -> (x_hat float64 [T, H] as the experts see it, sx float64 [T]).

    'mxfp8' applies the in-layer MX-32 quantisation of the bf16 input.
    """
    x = inp["x"]
    T = x.shape[0]
    if fmt in ("f32", "bf16"):
        return _decode_plain(x, fmt), np.ones(T)
    if fmt in ("mxfp8", "mxfp4"):
        xf = bf16_bits_to_f64(x).astype(np.float32)
        sc, q = mx_quantize(xf)
        return mx_dequantize(sc, q), np.ones(T)
    if fmt == "a8w8":
        return e4m3_decode(x), np.asarray(inp["x_scale"], dtype=np.float32).astype(np.float64)
    raise ValueError(fmt)


def gate_input(inp, fmt):
    """The layer input as real numbers (before any in-layer quantisation)."""
    if fmt == "a8w8":
        return e4m3_decode(inp["x"]) * np.asarray(inp["x_scale"], np.float32).astype(np.float64)[:, None]
    return _decode_plain(inp["x"], fmt)


def router_logits(inp, fmt):
    """Router logits l = x . Wr^T in float64 from the layer input as real
    numbers (a8w8: codes times the token's scale; MX formats: the bf16 input
    before its in-layer quantisation) and the router projection Wr [E, H]
    (fp32 for the f32 format, else bf16) -- the projection in front of the
    routing (vLLM PR 65207, Purpose, commit 1)."""
    wr = inp["router_w"]
    W = np.asarray(wr, np.float32).astype(np.float64) if fmt == "f32" else bf16_bits_to_f64(wr)
    return gate_input(inp, fmt) @ W.T


def gate(x, g):
    """gamma_t = sigmoid(sum_h x_th g_h), the dot product in float64."""
    z = np.asarray(x, np.float64) @ np.asarray(g, np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def _weights(w13, w2, s13, s2, fmt):
    if fmt in ("f32", "bf16"):
        return _decode_plain(w13, fmt), _decode_plain(w2, fmt), 1.0, 1.0
    if fmt == "mxfp8":
        return mx_dequantize(s13, w13), mx_dequantize(s2, w2), 1.0, 1.0
    if fmt == "mxfp4":
        return mx4_dequantize(s13, w13), mx4_dequantize(s2, w2), 1.0, 1.0
    if fmt == "a8w8":
        return e4m3_decode(w13), e4m3_decode(w2), float(np.float32(s13)), float(np.float32(s2))
    raise ValueError(fmt)


def expert_weights(inp, fmt, e):
    """Decoded routed expert e: (W13 [2I, H], W2 [H, I], scale13, scale2)."""
    s13 = inp.get("w13_scale")
    s2 = inp.get("w2_scale")
    return _weights(inp["w13"][e], inp["w2"][e],
                    None if s13 is None else s13[e], None if s2 is None else s2[e], fmt)


def shared_weights(inp, fmt):
    """Decoded shared expert: (Ws13 [2I_s, H], Ws2 [H, I_s], scale13, scale2)."""
    s13 = inp.get("ws13_scale")
    s2 = inp.get("ws2_scale")
    if fmt == "a8w8":
        s13 = np.asarray(s13).reshape(-1)[0]
        s2 = np.asarray(s2).reshape(-1)[0]
    return _weights(inp["ws13"], inp["ws2"], s13, s2, fmt)


def quantize_h(h, fmt):
    """Stage-1 output quantisation -> (h_tilde float64, row scale float64 [n])."""
    n = h.shape[0]
    if fmt == "f32":
        return h.astype(np.float32).astype(np.float64), np.ones(n)
    hb = bf16_bits_to_f64(round_to_bf16_bits(h))
    if fmt == "bf16":
        return hb, np.ones(n)
    if fmt in ("mxfp8", "mxfp4"):
        sc, q = mx_quantize(hb.astype(np.float32))
        return mx_dequantize(sc, q), np.ones(n)
    if fmt == "a8w8":
        s, q = row_quantize_e4m3(hb.astype(np.float32))
        return e4m3_decode(q), s.astype(np.float64)
    raise ValueError(fmt)


def activation(g, act):
    """The gate activation in float64: 'silu' g / (1 + e^-g); 'gelu_tanh'
    g/2 * (1 + tanh(sqrt(2/pi) * (g + 0.044715 g^3)))."""
    if act == "silu":
        return g / (1.0 + np.exp(-g))
    if act == "gelu_tanh":
        return 0.5 * g * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (g + 0.044715 * g ** 3)))
    raise ValueError(act)


def _f64(v):
    return None if v is None else np.asarray(v, dtype=np.float32).astype(np.float64)


def expert_mlp(xr, sx, W13, W2, s13, s2, fmt, intermediates=False, b13=None, b2=None, act="silu"):
    """One gated expert on rows xr [n, H] with per-row input scale sx [n]
    (optional fp32 biases b13 [2I], b2 [H]; act 'silu' or 'gelu_tanh')."""
    I = W2.shape[1]
    a = (xr @ W13.T) * sx[:, None] * s13
    if b13 is not None:
        a = a + _f64(b13)[None, :]
    g, u = a[:, :I], a[:, I:]
    h = activation(g, act) * u
    ht, sh = quantize_h(h, fmt)
    o = (ht @ W2.T) * sh[:, None] * s2
    if b2 is not None:
        o = o + _f64(b2)[None, :]
    if intermediates:
        return o, {"a": a, "h": h, "h_tilde": ht, "h_scale": sh}
    return o


def _expert_bias(inp, e):
    """(b13, b2) of routed expert e, or of the shared expert for e = None."""
    if e is None:
        return inp.get("bs13"), inp.get("bs2")
    b13, b2 = inp.get("b13"), inp.get("b2")
    return (None if b13 is None else b13[e]), (None if b2 is None else b2[e])


def route_layer(inp, prm, gamma=None, n_pseudo=0):
    """Routing of the layer (ids, weights) with the layer's parameters; the
    logits are the input's, or, when the layer is given its router projection
    instead, router_logits rounded to fp32 (the logits' type in the layer)."""
    logits = inp.get("logits")
    if logits is None:
        logits = router_logits(inp, prm.fmt).astype(np.float32)
    return route(logits, topk=prm.topk, score=prm.score, bias=inp.get("bias"),
                 n_group=prm.n_group, topk_group=prm.topk_group,
                 group_score_topk=prm.group_score_topk, renormalize=prm.renormalize,
                 routed_scaling_factor=prm.routed_scaling_factor,
                 n_pseudo=n_pseudo, gamma=gamma)


def moe_layer(inp, prm, tokens=None):
    """Full layer output for all tokens, or for the listed token indices.

    prm carries T, H, E, I, I_s, topk, score, n_group, topk_group,
    group_score_topk, renormalize, routed_scaling_factor, fmt and gated.
    Returns dict(y float64 [n, H], ids, w, gamma, tokens).
    """
    fmt = prm.fmt
    T = inp["x"].shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    xh, sx = decode_activations(inp, fmt)
    if prm.gated and inp.get("gate_w") is not None:
        gw = _decode_plain(inp["gate_w"], "f32" if fmt == "f32" else "bf16")
        gamma = gate(gate_input(inp, fmt), gw)
    else:
        gamma = np.ones(T)
    ids, w = route_layer(inp, prm)
    y = np.zeros((tokens.size, prm.H))
    sel_ids = ids[tokens]
    sel_w = w[tokens]
    act = getattr(prm, "activation", "silu")
    for e in np.unique(sel_ids):
        rows, slots = np.nonzero(sel_ids == e)
        W13, W2, s13, s2 = expert_weights(inp, fmt, int(e))
        b13, b2 = _expert_bias(inp, int(e))
        t = tokens[rows]
        o = expert_mlp(xh[t], sx[t], W13, W2, s13, s2, fmt, b13=b13, b2=b2, act=act)
        np.add.at(y, rows, sel_w[rows, slots][:, None] * o)
    if prm.I_s > 0:
        Ws13, Ws2, s13, s2 = shared_weights(inp, fmt)
        b13, b2 = _expert_bias(inp, None)
        o = expert_mlp(xh[tokens], sx[tokens], Ws13, Ws2, s13, s2, fmt, b13=b13, b2=b2, act=act)
        y += gamma[tokens][:, None] * o
    return {"y": y, "ids": ids, "w": w, "gamma": gamma, "tokens": tokens}


def stage1_reference(inp, prm, e, token_rows):
    """Stage-1 intermediate (h_tilde and row scale) of expert e on the given
    tokens; e == E denotes the whole shared expert."""
    fmt = prm.fmt
    xh, sx = decode_activations(inp, fmt)
    if e == prm.E:
        W13, W2, s13, s2 = shared_weights(inp, fmt)
        b13, b2 = _expert_bias(inp, None)
    else:
        W13, W2, s13, s2 = expert_weights(inp, fmt, e)
        b13, b2 = _expert_bias(inp, e)
    _, inter = expert_mlp(xh[token_rows], sx[token_rows], W13, W2, s13, s2, fmt, intermediates=True,
                          b13=b13, b2=b2, act=getattr(prm, "activation", "silu"))
    return inter
