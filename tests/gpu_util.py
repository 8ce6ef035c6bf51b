"""Helpers shared by the GPU parity tests (not collected by pytest)."""

import numpy as np
import torch

import oracle
import workloads

# Output tolerances: max |out - y_ref| <= TOL * RMS(y_ref), y_ref unrounded.
TOL = {"f32": 1e-5, "bf16": 2e-2, "mxfp8": 6e-2, "a8w8": 6e-2}

_cache = {}


def inputs(cfg, device):
    """Seeded inputs on the device (cached per config)."""
    key = (cfg, str(device))
    if key not in _cache:
        if len(_cache) > 3:
            _cache.clear()
            torch.cuda.empty_cache()
        _cache[key] = workloads.generate(cfg, device=device)
    return _cache[key]


def run_forward(cfg, inp, mode="auto", block_m=0, out_dtype=None):
    import routed_shared_experts_amd as m
    layer = m.MoeLayer(cfg, inp, shared_mode=mode, block_m=block_m, out_dtype=out_dtype)
    out = layer.forward()
    torch.cuda.synchronize()
    return out, layer


def compare(cfg, out, inp, tokens=None, lazy=False):
    """Oracle output for ``tokens`` (all when None); returns (err/rms, floor/rms)."""
    host = workloads.to_host(inp, lazy_weights=lazy)
    r = oracle.moe_layer(host, cfg, tokens=tokens)
    y = r["y"]
    got = out.float().cpu().numpy().astype(np.float64)
    if tokens is not None:
        got = got[np.asarray(tokens)]
    rms = np.sqrt((y ** 2).mean())
    err = np.abs(got - y).max()
    return err / rms, rounding_floor(y, out.dtype) / rms, r


def rounding_floor(y, dtype):
    """Largest error one correct rounding of y to the output type can make:
    half an ulp in the binade of max |y| (bf16: 8 significant bits)."""
    top = 2.0 ** np.floor(np.log2(np.abs(y).max()))
    return top * (2.0 ** -24 if dtype == torch.float32 else 2.0 ** -8)


def assert_close(cfg, out, inp, tokens=None, lazy=False):
    rel, floor, r = compare(cfg, out, inp, tokens, lazy)
    assert np.isfinite(rel)
    assert rel <= TOL[cfg.fmt], f"{cfg.name}: max|err|/rms = {rel:.3e} > {TOL[cfg.fmt]} (floor {floor:.3e})"
    return rel, floor, r
