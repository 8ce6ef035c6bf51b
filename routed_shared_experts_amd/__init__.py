"""Python binding of the fused routed + shared-expert MoE layer for MI355X.

Thin ctypes wrapper over ``libmoe.so`` (built from ``csrc/`` with hipcc for
gfx950).  It only marshals arguments: torch tensors are passed as raw device
pointers together with the current HIP stream; every step of the layer runs
in the library's kernels.  Importing this package raises if the library has
not been built; there is no fallback implementation.

The entry points mirror the C ABI in ``include/moe.h``: ``moe_route``,
``shared_gate_dot``, ``moe_quant_mx``, ``moe_sort_tokens``, ``moe_stage1``,
``moe_stage2_accum`` and the fused ``moe_forward``, plus ``moe_validate``,
``moe_workspace_bytes``, ``moe_sort_capacity``, ``moe_query_feature`` and
``moe_status_str``; ``moe_pack_weights`` / ``moe_pack_mx_scales`` convert
row-major weights to the tiled layout the GEMM kernels read.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

# ---- enums (values fixed by include/moe.h) ----
MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_FP4_E2M1 = 0, 1, 2, 3
MOE_SCALE_NONE, MOE_SCALE_PER_ROW, MOE_SCALE_PER_EXPERT, MOE_SCALE_MX32 = 0, 1, 2, 3
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_SHARED_NONE, MOE_SHARED_PSEUDO, MOE_SHARED_AUX, MOE_SHARED_AUTO = 0, 1, 2, 3
MOE_STAGE2_STORE, MOE_STAGE2_ACCUMULATE = 0, 1
MOE_LAYOUT_ROW_MAJOR, MOE_LAYOUT_TILED = 0, 1
MOE_ACT_SILU, MOE_ACT_GELU_TANH = 0, 1
(MOE_FEATURE_ACCUMULATE_OUTPUT, MOE_FEATURE_PSEUDO_SHARED, MOE_FEATURE_AUX_STREAM,
 MOE_FEATURE_MXFP8, MOE_FEATURE_A8W8, MOE_FEATURE_F32, MOE_FEATURE_BF16, MOE_FEATURE_MXFP4,
 MOE_FEATURE_EXPERT_BIAS, MOE_FEATURE_GELU_TANH, MOE_FEATURE_ROUTER_GEMM) = 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11
ACTIVATIONS = {"silu": MOE_ACT_SILU, "gelu_tanh": MOE_ACT_GELU_TANH}

SHARED_MODES = {"none": MOE_SHARED_NONE, "pseudo": MOE_SHARED_PSEUDO, "aux": MOE_SHARED_AUX,
                "auto": MOE_SHARED_AUTO}

# Exported symbols, in the order of include/moe.h.
EXPORTS = ["moe_validate", "moe_workspace_bytes", "moe_forward", "moe_forward_noalloc", "moe_route", "moe_router_logits",
           "shared_gate_dot",
           "moe_quant_mx", "moe_sort_capacity", "moe_sort_scratch_bytes", "moe_pack_weights", "moe_pack_mx_scales",
           "moe_sort_tokens", "moe_stage1", "moe_stage2_accum", "moe_query_feature", "moe_status_str",
           "moe_last_hip_error"]

c_void_p, c_int32, c_float, c_size_t = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t


class MoeWeights(ctypes.Structure):
    _fields_ = [("w13", c_void_p), ("w2", c_void_p), ("w13_scale", c_void_p), ("w2_scale", c_void_p),
                ("dtype", c_int32), ("scale", c_int32), ("layout", c_int32), ("b13", c_void_p),
                ("b2", c_void_p)]


class MoeForwardArgs(ctypes.Structure):
    _fields_ = [("T", c_int32), ("H", c_int32), ("E", c_int32), ("I", c_int32), ("I_s", c_int32),
                ("topk", c_int32), ("score", c_int32), ("n_group", c_int32), ("topk_group", c_int32),
                ("group_score_topk", c_int32), ("renormalize", c_int32),
                ("routed_scaling_factor", c_float), ("logits", c_void_p), ("bias", c_void_p),
                ("x", c_void_p), ("x_dtype", c_int32), ("x_row_scale", c_void_p),
                ("routed", MoeWeights), ("shared", MoeWeights), ("gate_w", c_void_p),
                ("shared_mode", c_int32), ("block_m", c_int32), ("out", c_void_p),
                ("out_dtype", c_int32), ("timing_events", c_void_p), ("activation", c_int32),
                ("router_w", c_void_p)]


class MoeStageArgs(ctypes.Structure):
    _fields_ = [("T", c_int32), ("H", c_int32), ("E", c_int32), ("I", c_int32), ("I_s", c_int32),
                ("n_pseudo", c_int32), ("k_total", c_int32), ("routed", MoeWeights),
                ("shared", MoeWeights), ("x", c_void_p), ("x_scale", c_void_p), ("dense", c_int32),
                ("block_m", c_int32), ("max_blocks", c_int32), ("sorted_pair_ids", c_void_p),
                ("block_expert", c_void_p), ("num_blocks", c_void_p), ("h", c_void_p),
                ("h_scale", c_void_p), ("pair_w", c_void_p), ("gamma", c_void_p), ("acc", c_void_p),
                ("pair_out", c_void_p), ("out", c_void_p), ("out_dtype", c_int32), ("mode", c_int32),
                ("counters", c_void_p), ("expected_arrivals", c_int32), ("addend_ready", c_void_p),
                ("activation", c_int32)]


class MoeError(RuntimeError):
    pass


def _load():
    # torch ships its own HIP runtime under the same soname as /opt/rocm's; load
    # it first so that the process has one runtime, the one torch's device
    # memory and streams belong to (loading libmoe.so first would bind both to
    # /opt/rocm's copy)
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()' "
            "or python routed_shared_experts_amd/build.py); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    sig = {
        "moe_validate": (c_int32, [P(MoeForwardArgs)]),
        "moe_workspace_bytes": (c_size_t, [P(MoeForwardArgs)]),
        "moe_forward": (c_int32, [P(MoeForwardArgs), c_void_p, c_size_t, c_void_p, c_void_p, c_void_p,
                                  c_void_p]),
        "moe_forward_noalloc": (c_int32, [P(MoeForwardArgs), c_void_p, c_void_p, c_void_p, c_void_p]),
        "moe_route": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                c_int32, c_int32, c_float, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
        "moe_router_logits": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                        c_void_p, c_void_p]),
        "shared_gate_dot": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_int32, c_void_p,
                                      c_void_p]),
        "moe_quant_mx": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
        "moe_sort_capacity": (c_int32, [c_int32, c_int32, c_int32, c_int32]),
        "moe_sort_scratch_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
        "moe_pack_weights": (c_int32, [c_void_p, c_void_p, ctypes.c_int64, c_int32, c_void_p]),
        "moe_pack_mx_scales": (c_int32, [c_void_p, c_void_p, ctypes.c_int64, c_int32, c_void_p]),
        "moe_sort_tokens": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p,
                                      c_size_t, c_void_p]),
        "moe_stage1": (c_int32, [P(MoeStageArgs), c_void_p]),
        "moe_stage2_accum": (c_int32, [P(MoeStageArgs), c_void_p]),
        "moe_query_feature": (c_int32, [c_int32]),
        "moe_status_str": (ctypes.c_char_p, [c_int32]),
        "moe_last_hip_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def lib():
    return _lib


def moe_status_str(status):
    return _lib.moe_status_str(int(status)).decode()


def _check(status, what):
    if status != MOE_OK:
        detail = f" ({_lib.moe_last_hip_error().decode()})" if status == MOE_ERR_HIP else ""
        raise MoeError(f"{what} failed: {moe_status_str(status)}{detail}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def moe_query_feature(feature):
    return int(_lib.moe_query_feature(int(feature)))


def moe_sort_capacity(T, k_total, n_experts, block_m):
    return int(_lib.moe_sort_capacity(T, k_total, n_experts, block_m))


def moe_validate(args):
    return int(_lib.moe_validate(ctypes.byref(args)))


def moe_workspace_bytes(args):
    return int(_lib.moe_workspace_bytes(ctypes.byref(args)))


def moe_router_logits(x, router_w, logits, x_row_scale=None, stream=None):
    """logits [T, E] fp32 = x . router_w^T (x fp32 / bf16 / float8_e4m3fn codes
    with x_row_scale; router_w [E, H] fp32 for fp32 x, else bf16)."""
    import torch
    T, H = x.shape
    E = router_w.shape[0]
    xdt = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}.get(x.dtype, MOE_FP8_E4M3)
    st = _lib.moe_router_logits(_ptr(x), xdt, _ptr(x_row_scale), _ptr(router_w), T, H, E, _ptr(logits),
                                _stream(stream))
    _check(st, "moe_router_logits")


def moe_route(logits, topk_ids, topk_w, *, topk, bias=None, n_group=1, topk_group=1, group_score_topk=2,
              score=MOE_SCORE_SOFTMAX, renormalize=True, routed_scaling_factor=1.0, n_pseudo=0,
              gamma=None, stream=None):
    T, E = logits.shape
    st = _lib.moe_route(_ptr(logits), _ptr(bias), T, E, topk, n_group, topk_group, group_score_topk, score,
                        int(bool(renormalize)), float(routed_scaling_factor), n_pseudo, _ptr(gamma),
                        _ptr(topk_ids), _ptr(topk_w), _stream(stream))
    _check(st, "moe_route")


def shared_gate_dot(x, g, gate_out, apply_sigmoid=True, stream=None):
    import torch
    dt = MOE_F32 if x.dtype == torch.float32 else MOE_BF16
    T, H = x.shape
    st = _lib.shared_gate_dot(_ptr(x), dt, _ptr(g), T, H, int(bool(apply_sigmoid)), _ptr(gate_out),
                              _stream(stream))
    _check(st, "shared_gate_dot")


def moe_quant_mx(x, codes, scales, stream=None):
    T, H = x.shape
    st = _lib.moe_quant_mx(_ptr(x), T, H, _ptr(codes), _ptr(scales), _stream(stream))
    _check(st, "moe_quant_mx")


def moe_pack_weights(src, dst=None, stream=None):
    """Tiled copy of a row-major weight tensor whose last dimension is K (any
    leading dimensions: stacked matrices); returns dst (new if None)."""
    import torch
    dst = torch.empty_like(src) if dst is None else dst
    row_bytes = src.shape[-1] * src.element_size()
    rows = src.numel() * src.element_size() // row_bytes
    _check(_lib.moe_pack_weights(_ptr(src), _ptr(dst), rows, row_bytes, _stream(stream)), "moe_pack_weights")
    return dst


def moe_pack_mx_scales(src, dst=None, stream=None):
    """Tiled copy of a row-major uint8 MX32 scale tensor (last dimension =
    scale bytes per row); returns dst (new if None)."""
    import torch
    dst = torch.empty_like(src) if dst is None else dst
    sb = src.shape[-1]
    _check(_lib.moe_pack_mx_scales(_ptr(src), _ptr(dst), src.numel() // sb, sb, _stream(stream)),
           "moe_pack_mx_scales")
    return dst


def moe_sort_scratch_bytes(T, k_total, n_experts):
    return int(_lib.moe_sort_scratch_bytes(T, k_total, n_experts))


def moe_sort_tokens(topk_ids, n_experts, block_m, capacity, sorted_pair_ids, block_expert, counts, offsets,
                    num_blocks, scratch=None, zero=None, stream=None):
    T, k_total = topk_ids.shape
    zb = 0 if zero is None else zero.numel() * zero.element_size()
    sb = 0 if scratch is None else scratch.numel() * scratch.element_size()
    st = _lib.moe_sort_tokens(_ptr(topk_ids), T, k_total, n_experts, block_m, capacity, _ptr(sorted_pair_ids),
                              _ptr(block_expert), _ptr(counts), _ptr(offsets), _ptr(num_blocks), _ptr(scratch),
                              sb, _ptr(zero), zb, _stream(stream))
    _check(st, "moe_sort_tokens")


def moe_stage1(args, stream=None):
    _check(_lib.moe_stage1(ctypes.byref(args), _stream(stream)), "moe_stage1")


def moe_stage2_accum(args, stream=None):
    _check(_lib.moe_stage2_accum(ctypes.byref(args), _stream(stream)), "moe_stage2_accum")


def moe_forward(args, workspace, main_stream=None, aux_stream=None, ev_fork=None, ev_ready=None):
    """Run the layer; ``workspace`` is a uint8 device tensor of at least
    ``moe_workspace_bytes(args)`` bytes.  ev_fork / ev_ready are raw hipEvent
    handles (ints) or None."""
    aux = ctypes.c_void_p(aux_stream.cuda_stream) if aux_stream is not None else None
    st = _lib.moe_forward(ctypes.byref(args), _ptr(workspace), workspace.numel(), _stream(main_stream), aux,
                          ctypes.c_void_p(ev_fork) if ev_fork else None,
                          ctypes.c_void_p(ev_ready) if ev_ready else None)
    _check(st, "moe_forward")


MOE_NOALLOC_SCRATCH_BYTES = 64 << 20  # include/moe.h


def moe_forward_noalloc(args, main_stream=None, aux_stream=None, ev_fork=None, ev_ready=None):
    """Run the layer on the library's own per-device scratch (no workspace,
    nothing allocated); raises MoeError with MOE_ERR_WORKSPACE when the
    request needs more than MOE_NOALLOC_SCRATCH_BYTES."""
    aux = ctypes.c_void_p(aux_stream.cuda_stream) if aux_stream is not None else None
    st = _lib.moe_forward_noalloc(ctypes.byref(args), _stream(main_stream), aux,
                                  ctypes.c_void_p(ev_fork) if ev_fork else None,
                                  ctypes.c_void_p(ev_ready) if ev_ready else None)
    _check(st, "moe_forward_noalloc")


from .layer import (FORMATS, weights_struct, forward_args, pack_weights, MoeLayer)  # noqa: E402,F401
