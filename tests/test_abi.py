"""The C ABI without a GPU: the library loads, exports every function the
header declares, the ctypes structs match the C layout, and the pure-host
validation rejects what it must (no compute calls)."""

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import routed_shared_experts_amd as m
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)


def test_header_declares_the_binding_exports():
    decl = set(_declared_functions())
    assert decl == set(m.EXPORTS), decl ^ set(m.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True, text=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [f for f in _declared_functions() if f not in syms]
    assert not missing, missing
    for f in _declared_functions():
        assert hasattr(m.lib(), f)


def _c_layout(struct, fields):
    prog = "#include <cstdio>\n#include <cstddef>\n#include \"moe.h\"\nint main(){\n"
    prog += f'printf("%zu\\n", sizeof({struct}));\n'
    for f in fields:
        prog += f'printf("%zu\\n", offsetof({struct}, {f}));\n'
    prog += "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "l.cpp"), os.path.join(d, "l")
        open(src, "w").write(prog)
        subprocess.run(["g++", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I",
                        "/opt/rocm/include", src, "-o", exe], check=True, capture_output=True)
        vals = [int(v) for v in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    return vals[0], vals[1:]


@pytest.mark.parametrize("cls,name", [(m.MoeForwardArgs, "moe_forward_args"),
                                      (m.MoeStageArgs, "moe_stage_args"),
                                      (m.MoeWeights, "moe_weights")])
def test_struct_layout_matches_header(cls, name):
    fields = [f for f, _ in cls._fields_]
    size, offs = _c_layout(name, fields)
    assert size == ctypes.sizeof(cls)
    assert offs == [getattr(cls, f).offset for f in fields]


def test_status_strings_and_features():
    assert m.moe_status_str(m.MOE_ERR_WORKSPACE) == "MOE_ERR_WORKSPACE"
    for f in range(1, 8):
        assert m.moe_query_feature(f) == 1
    assert m.moe_query_feature(99) == 0


def test_sort_capacity():
    # T*k + min(E, T*k)*(BM-1), rounded up to BM
    cap = m.moe_sort_capacity(32, 9, 65, 16)
    assert cap % 16 == 0 and cap >= 288 + 65 * 15
    assert m.moe_sort_capacity(1, 1, 100, 64) == 64


class _Fake:
    """Stands in for a device tensor: an aligned fake address (never dereferenced)."""

    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


def _fake_inputs(cfg):
    keys = ["x", "x_scale", "logits", "bias", "gate_w", "w13", "w2", "w13_scale", "w2_scale", "ws13", "ws2",
            "ws13_scale", "ws2_scale"]
    return {k: _Fake(0x10000 * (i + 1)) for i, k in enumerate(keys)}


def _args(cfg, mode="auto", **over):
    inp = _fake_inputs(cfg)
    if cfg.bias_std == 0:
        inp["bias"] = None
    if not cfg.gated:
        inp["gate_w"] = None
    if cfg.fmt not in ("mxfp8", "a8w8"):
        for k in ("w13_scale", "w2_scale", "ws13_scale", "ws2_scale"):
            inp[k] = None
    if cfg.fmt != "a8w8":
        inp["x_scale"] = None
    a = m.forward_args(cfg, inp, _Fake(0x900000), mode)
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_validate_accepts_every_workload(name):
    cfg = workloads.CONFIGS[name]
    for mode in ("auto", "pseudo", "aux"):
        a = _args(cfg, mode)
        assert m.moe_validate(a) == m.MOE_OK, (name, mode)
        assert m.moe_workspace_bytes(a) > 0


def test_validate_rejections():
    c = workloads.CONFIGS["decode_bf16"]
    assert m.moe_validate(_args(c, H=2000)) == m.MOE_ERR_INVALID_ARG           # H % 64
    assert m.moe_validate(_args(c, topk=65)) == m.MOE_ERR_INVALID_ARG          # k > E
    assert m.moe_validate(_args(c, n_group=3)) == m.MOE_ERR_INVALID_ARG        # E % n_group
    assert m.moe_validate(_args(c, n_group=16, topk_group=1)) == m.MOE_ERR_INVALID_ARG  # k > Gk*E/G
    assert m.moe_validate(_args(c, topk_group=2)) == m.MOE_ERR_INVALID_ARG     # Gk > G
    assert m.moe_validate(_args(c, block_m=48)) == m.MOE_ERR_INVALID_ARG
    assert m.moe_validate(_args(c, x=ctypes.c_void_p(0x10008))) == m.MOE_ERR_INVALID_ARG  # misaligned
    assert m.moe_validate(_args(c, out=None)) == m.MOE_ERR_INVALID_ARG
    assert m.moe_validate(_args(c, x_dtype=m.MOE_F32)) == m.MOE_ERR_UNSUPPORTED
    assert m.moe_validate(_args(c, shared_mode=m.MOE_SHARED_NONE)) == m.MOE_ERR_INVALID_ARG  # I_s > 0
    mx = workloads.CONFIGS["mxfp8"]
    assert m.moe_validate(_args(mx, I=1552)) == m.MOE_ERR_INVALID_ARG          # MX needs K % 32 (and the K tile)
    # shared weights in another format: pseudo fusion unsupported, auto falls back to aux
    a = _args(mx, "pseudo")
    a.shared.dtype, a.shared.scale = m.MOE_BF16, m.MOE_SCALE_NONE
    assert m.moe_validate(a) == m.MOE_ERR_UNSUPPORTED
    q = workloads.CONFIGS["a8w8_large"]
    assert m.moe_validate(_args(q, "pseudo", I_s=4096)) == m.MOE_ERR_UNSUPPORTED  # row scale needs m == 1
    assert m.moe_validate(_args(q, "aux", I_s=4096)) == m.MOE_OK
    assert m.moe_validate(_args(q, x_row_scale=None)) == m.MOE_ERR_INVALID_ARG
    # the kernels read tiled weights only
    a = _args(c)
    a.routed.layout = m.MOE_LAYOUT_ROW_MAJOR
    assert m.moe_validate(a) == m.MOE_ERR_UNSUPPORTED
    a = _args(c, "aux")
    a.shared.layout = 7
    assert m.moe_validate(a) == m.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ["decode_bf16", "a8w8_large"])
def test_empty_batch_is_a_valid_no_op(name):
    """T = 0: valid with NULL logits / x / out / row scales, a positive
    workspace size, and moe_forward returns MOE_OK without a HIP call (no
    workspace, streams or events needed) -- so it runs without a GPU."""
    c = workloads.CONFIGS[name]
    for mode in ("pseudo", "aux"):
        a = _args(c, mode, T=0, logits=None, x=None, out=None, x_row_scale=None)
        assert m.moe_validate(a) == m.MOE_OK
        assert m.moe_workspace_bytes(a) > 0
        assert m.lib().moe_forward(ctypes.byref(a), None, 0, None, None, None, None) == m.MOE_OK
    assert m.moe_validate(_args(c, T=-1)) == m.MOE_ERR_INVALID_ARG
    assert m.moe_validate(_args(c, x=None)) == m.MOE_ERR_INVALID_ARG  # T > 0 needs its inputs


def test_forward_rejects_without_launching():
    """Invalid requests and a too-small workspace return before any HIP call,
    so they work on a machine without a GPU."""
    c = workloads.CONFIGS["decode_bf16"]
    a = _args(c)
    st = m.lib().moe_forward(ctypes.byref(a), ctypes.c_void_p(0x4000000), 1024, None, None, None, None)
    assert st == m.MOE_ERR_WORKSPACE
    st = m.lib().moe_forward(ctypes.byref(a), ctypes.c_void_p(0x4000010), 1 << 40, None, None, None, None)
    assert st == m.MOE_ERR_WORKSPACE  # misaligned workspace
    a_aux = _args(c, "aux")
    need = m.moe_workspace_bytes(a_aux)
    st = m.lib().moe_forward(ctypes.byref(a_aux), ctypes.c_void_p(0x4000000), need, None, None, None, None)
    assert st == m.MOE_ERR_INVALID_ARG  # aux mode needs two distinct streams and events
    bad = _args(c, topk=0)
    assert m.lib().moe_forward(ctypes.byref(bad), None, 0, None, None, None, None) == m.MOE_ERR_INVALID_ARG


def test_step_entry_points_reject_bad_arguments():
    L = m.lib()
    assert L.moe_route(None, None, 4, 8, 2, 1, 1, 2, 0, 1, 1.0, 0, None, None, None, None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_route(ctypes.c_void_p(0x1000), None, 4, 8, 9, 1, 1, 2, 0, 1, 1.0, 0, None,
                       ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000), None) == m.MOE_ERR_INVALID_ARG
    assert L.shared_gate_dot(ctypes.c_void_p(0x1000), m.MOE_FP8_E4M3, ctypes.c_void_p(0x2000), 1, 64, 1,
                             ctypes.c_void_p(0x3000), None) == m.MOE_ERR_UNSUPPORTED
    assert L.moe_quant_mx(ctypes.c_void_p(0x1000), 2, 48, ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000),
                          None) == m.MOE_ERR_INVALID_ARG  # H % 32
    p = ctypes.c_void_p(0x1000)
    assert L.moe_sort_tokens(p, 4, 2, 8, 16, 16, p, p, p, p, p, None, 0, None, 0, None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_sort_tokens(p, 4, 2, 600, 16, 4096, p, p, p, p, p, None, 0, None, 0, None) == m.MOE_ERR_INVALID_ARG
    big = m.moe_sort_scratch_bytes(8192, 9, 257)
    assert big == 72 * 257 * 4 and m.moe_sort_scratch_bytes(32, 9, 65) == 0
    cap = m.moe_sort_capacity(8192, 9, 257, 128)
    assert L.moe_sort_tokens(p, 8192, 9, 257, 128, cap, p, p, p, p, p, p, big - 4, None, 0,
                             None) == m.MOE_ERR_WORKSPACE
    # pack: rows % 16, row_bytes % 128, alignment, overlapping buffers
    src, dst = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    assert L.moe_pack_weights(src, dst, 24, 256, None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights(src, dst, 32, 200, None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights(ctypes.c_void_p(0x100008), dst, 32, 256, None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights(src, ctypes.c_void_p(0x100000 + 32 * 256 - 16), 32, 256, None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights(src, dst, 0, 256, None) == m.MOE_OK  # nothing to do, no launch
    assert L.moe_pack_mx_scales(src, dst, 16, 6, None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_pack_mx_scales(src, dst, 8, 8, None) == m.MOE_ERR_INVALID_ARG
    sa = m.MoeStageArgs()
    assert L.moe_stage1(ctypes.byref(sa), None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_stage2_accum(None, None) == m.MOE_ERR_INVALID_ARG


def test_router_weights_replace_the_logits_input():
    """With router weights the logits input may be NULL; the router GEMM's
    shape and pointer rules are checked before any launch."""
    c = workloads.CONFIGS["decode_bf16"]
    rw = ctypes.c_void_p(0x7000000)
    a = _args(c, logits=None, router_w=rw)
    assert m.moe_validate(a) == m.MOE_OK
    assert m.moe_workspace_bytes(a) >= m.moe_workspace_bytes(_args(c)) + c.T * c.E * 4
    assert m.moe_validate(_args(c, logits=None)) == m.MOE_ERR_INVALID_ARG          # neither
    assert m.moe_validate(_args(c, logits=None, router_w=ctypes.c_void_p(0x7000008))) == m.MOE_ERR_INVALID_ARG
    L = m.lib()
    p = ctypes.c_void_p(0x1000)
    assert L.moe_router_logits(p, m.MOE_BF16, None, p, 4, 96, 8, p, None) == m.MOE_ERR_INVALID_ARG   # H % 64
    assert L.moe_router_logits(p, m.MOE_F32, None, p, 4, 80, 8, p, None) == m.MOE_ERR_INVALID_ARG    # H % 32
    assert L.moe_router_logits(p, m.MOE_BF16, None, p, 4, 128, 513, p, None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_router_logits(p, m.MOE_FP8_E4M3, None, p, 4, 128, 8, p, None) == m.MOE_ERR_INVALID_ARG  # scale
    assert L.moe_router_logits(p, m.MOE_FP4_E2M1, None, p, 4, 128, 8, p, None) == m.MOE_ERR_UNSUPPORTED
    assert L.moe_router_logits(None, m.MOE_BF16, None, None, 0, 128, 8, None, None) == m.MOE_OK      # empty
    assert m.moe_query_feature(m.MOE_FEATURE_ROUTER_GEMM) == 1
