"""CPU oracle for the fused routed + shared-expert MoE layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (no kernels, headers, helpers, tables or constant generators) and it
imports nothing from the ``routed_shared_experts_amd`` package.

It is a plain, slow, obviously-correct restatement of what the layer computes,
in float64 wherever the pages leave the precision open, using numpy.  Each
function cites the passage it follows.  The pages are five public pull-request
discussions:

* vLLM PR 61503, "Fused heterogeneous MoE support" (FHMoE) -- routed and
  shared experts in one fused op, with a multi-stream fallback (Overview).
* vLLM PR 65207, shared-expert output accumulated in the AITER stage-2 GEMM
  epilogue (Purpose, commits 1-3; Dependencies; the review measurements).
* AITER PR 6106, "[Triton/Gluon] Add per token scale to a8w8 moe gemm"
  (Technical Details).
* vLLM PR 56789, shared-expert sigmoid gate as a tiny dot product (Summary,
  Commits, Testing).
* SGLang PR 27057, "[AMD] move shared expert check function to quark"
  (Modifications, item 1).

Parity status per function (what pins it, in ``tests/test_oracle_*.py``):

* codecs (bf16, e4m3fn, e8m0, MX-32, per-row e4m3, e2m1 / MXFP4): pinned --
  exhaustive code tables vs the OCP closed forms (the e2m1 table of the OCP MX
  specification as a golden file) and torch's float8/bfloat16 casts,
  brute-force nearest-code search, crafted MX blocks, the nibble order.
* spec_exp / spec_sigmoid: pinned -- exact special values, <= 2 ulp against
  float64 on a dense sweep, monotonicity.
* route: pinned -- definition checks on every token, exhaustive group-subset
  enumeration, closed-form equal-logit weights, torch.topk on tie-free inputs.
* sort_tokens: pinned -- independent stable argsort, invariants.
* gate / expert / layer: pinned -- torch float64 library routines on the
  E = 1 case, dense brute force with unselected weights zeroed, the
  shared-only and scale-folding identities.
* the fp8 expert chain (MXFP8 and a8w8: bf16 rounding of h, MX-32 or per-row
  quantisation of h, the row scale times the expert scale): pinned -- an
  independent torch float64 reference built from the format definitions with
  torch's float8_e4m3fn and bfloat16 casts, equal h codes and outputs, and
  planted mistakes in the oracle that the comparison catches.
* biased sigmoid routing weights: pinned -- closed-form weights
  sigmoid(l_j) / sum sigmoid(l_sel) * s on a case where the bias changes the
  selection, with and without groups.
"""

from .codecs import (
    bf16_bits_to_f64,
    round_to_bf16_bits,
    e4m3_decode,
    e4m3_encode_rne_sat,
    e8m0_decode,
    mx_quantize,
    mx_dequantize,
    row_quantize_e4m3,
    e2m1_decode,
    e2m1_unpack,
    mx4_dequantize,
)
from .specmath import spec_exp, spec_sigmoid
from .routing import route
from .sorting import sort_tokens
from .layer import (
    gate,
    router_logits,
    decode_activations,
    expert_weights,
    shared_weights,
    expert_mlp,
    activation,
    moe_layer,
    stage1_reference,
)

__all__ = [
    "bf16_bits_to_f64", "round_to_bf16_bits", "e4m3_decode", "e4m3_encode_rne_sat",
    "e8m0_decode", "mx_quantize", "mx_dequantize", "row_quantize_e4m3", "e2m1_decode", "e2m1_unpack",
    "mx4_dequantize",
    "spec_exp", "spec_sigmoid", "route", "sort_tokens", "gate", "router_logits",
    "decode_activations", "expert_weights", "shared_weights", "expert_mlp", "activation",
    "moe_layer", "stage1_reference",
]
