"""Argument marshalling for the fused layer: torch tensors -> ``moe_forward_args``.

Nothing here computes any part of the layer; it fills the C structs with
device pointers, owns the workspace tensor and the second stream / events the
aux-stream mode needs, and calls the library.
"""

import torch

from . import (MoeForwardArgs, MoeWeights, ACTIVATIONS, MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_FP4_E2M1, MOE_SCALE_NONE,
               MOE_SCALE_PER_EXPERT, MOE_SCALE_MX32, MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID,
               MOE_LAYOUT_TILED, SHARED_MODES, MOE_OK, MoeError, moe_validate, moe_workspace_bytes,
               moe_forward, moe_pack_weights, moe_pack_mx_scales, moe_status_str, _ptr)

# layer format -> (x dtype, weight dtype, weight scale kind, output dtype)
FORMATS = {
    "f32": (MOE_F32, MOE_F32, MOE_SCALE_NONE, MOE_F32),
    "bf16": (MOE_BF16, MOE_BF16, MOE_SCALE_NONE, MOE_BF16),
    "mxfp8": (MOE_BF16, MOE_FP8_E4M3, MOE_SCALE_MX32, MOE_BF16),
    "a8w8": (MOE_FP8_E4M3, MOE_FP8_E4M3, MOE_SCALE_PER_EXPERT, MOE_BF16),
    "mxfp4": (MOE_BF16, MOE_FP4_E2M1, MOE_SCALE_MX32, MOE_BF16),
}


def weights_struct(w13, w2, s13, s2, fmt, b13=None, b2=None):
    """Weight family struct; the tensors must already be in the tiled layout
    (b13, b2: optional fp32 biases)."""
    _, wdt, wsc, _ = FORMATS[fmt]
    return MoeWeights(_ptr(w13), _ptr(w2), _ptr(s13), _ptr(s2), wdt, wsc, MOE_LAYOUT_TILED, _ptr(b13), _ptr(b2))


def pack_weights(cfg, inp, stream=None):
    """Tiled copies of the layer's weight matrices (and MX32 scale matrices),
    made once at load time: {"w13", "w2", ["ws13", "ws2"], [scales]}.  Per-expert
    scales and every non-weight input are used as they are."""
    out = {}
    names = ["w13", "w2"] + (["ws13", "ws2"] if cfg.I_s > 0 else [])
    for n in names:
        out[n] = moe_pack_weights(inp[n], stream=stream)
        if cfg.fmt in ("mxfp8", "mxfp4"):
            out[n + "_scale"] = moe_pack_mx_scales(inp[n + "_scale"], stream=stream)
    return out


def forward_args(cfg, inp, out, shared_mode="auto", block_m=0, out_dtype=None):
    """Fill a MoeForwardArgs from a workload config and its input tensors
    (out_dtype: MOE_F32 or MOE_BF16; None = the format's own output type)."""
    xdt, _, _, odt = FORMATS[cfg.fmt]
    odt = odt if out_dtype is None else out_dtype
    a = MoeForwardArgs()
    a.T, a.H, a.E, a.I, a.I_s, a.topk = cfg.T, cfg.H, cfg.E, cfg.I, cfg.I_s, cfg.topk
    a.score = MOE_SCORE_SOFTMAX if cfg.score == "softmax" else MOE_SCORE_SIGMOID
    a.n_group, a.topk_group, a.group_score_topk = cfg.n_group, cfg.topk_group, cfg.group_score_topk
    a.renormalize = int(bool(cfg.renormalize))
    a.routed_scaling_factor = float(cfg.routed_scaling_factor)
    a.logits = _ptr(inp.get("logits"))
    a.router_w = _ptr(inp.get("router_w"))
    a.bias = _ptr(inp.get("bias"))
    a.x = _ptr(inp["x"])
    a.x_dtype = xdt
    a.x_row_scale = _ptr(inp.get("x_scale"))
    a.routed = weights_struct(inp["w13"], inp["w2"], inp.get("w13_scale"), inp.get("w2_scale"), cfg.fmt,
                              inp.get("b13"), inp.get("b2"))
    if cfg.I_s > 0:
        a.shared = weights_struct(inp["ws13"], inp["ws2"], inp.get("ws13_scale"), inp.get("ws2_scale"), cfg.fmt,
                                  inp.get("bs13"), inp.get("bs2"))
    a.activation = ACTIVATIONS[getattr(cfg, "activation", "silu")]
    a.gate_w = _ptr(inp.get("gate_w")) if cfg.gated else None
    a.shared_mode = SHARED_MODES[shared_mode] if cfg.I_s > 0 else SHARED_MODES["none"]
    a.block_m = block_m
    a.out = _ptr(out)
    a.out_dtype = odt
    return a


class MoeLayer:
    """One configured layer forward on the current device.

    Holds references to the input tensors and the tiled weight copies (so the
    pointers stay valid), the output tensor, the workspace, and, for the
    aux-stream mode, a second stream and two events.
    """

    def __init__(self, cfg, inp, shared_mode="auto", block_m=0, out=None, packed=None, out_dtype=None):
        """inp: the workload's tensors with row-major weights; packed: their
        tiled copies from pack_weights (made here when None); out_dtype:
        MOE_F32 or MOE_BF16 (None: the format's own output type)."""
        packed = pack_weights(cfg, inp) if packed is None else packed
        inp = dict(inp, **packed)
        self.cfg, self.inp = cfg, inp
        dev = inp["x"].device
        odt_c = FORMATS[cfg.fmt][3] if out_dtype is None else out_dtype
        odt = torch.float32 if odt_c == MOE_F32 else torch.bfloat16
        self.out = out if out is not None else torch.empty((cfg.T, cfg.H), dtype=odt, device=dev)
        self.args = forward_args(cfg, inp, self.out, shared_mode, block_m, odt_c)
        st = moe_validate(self.args)
        if st != MOE_OK:
            raise MoeError(f"moe_validate: {moe_status_str(st)}")
        self.ws_bytes = moe_workspace_bytes(self.args)
        self.workspace = torch.empty((self.ws_bytes,), dtype=torch.uint8, device=dev)
        self.aux_stream = torch.cuda.Stream(device=dev)   # default priority
        cur = torch.cuda.current_stream(dev)
        self.ev_fork = torch.cuda.Event()
        self.ev_ready = torch.cuda.Event()
        self.ev_fork.record(cur)     # materialise the events so their handles exist
        self.ev_ready.record(cur)

    def forward(self, stream=None):
        moe_forward(self.args, self.workspace, main_stream=stream, aux_stream=self.aux_stream,
                    ev_fork=self.ev_fork.cuda_event, ev_ready=self.ev_ready.cuda_event)
        return self.out
