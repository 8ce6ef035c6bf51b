"""Helpers shared by the GPU parity tests (not collected by pytest)."""

import numpy as np
import torch

import oracle
import workloads

# Output tolerances: max |out - y_ref| <= TOL * RMS(y_ref), y_ref unrounded.
TOL = {"f32": 1e-5, "bf16": 2e-2, "mxfp8": 6e-2, "mxfp4": 6e-2, "a8w8": 6e-2}

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


def auto_block_m(rows_per_expert):
    """The library's automatic block size: the smallest of 16/32/64 rows that
    holds 1.5x the mean rows per expert, else 128."""
    need = 1.5 * rows_per_expert
    for bm in (16, 32, 64):
        if need <= bm:
            return bm
    return 128


def stage2_reference(cfg, host, srt, ids, w, h_vals, h_scale, kt, shared=None):
    """Oracle stage 2 fed the GPU's own intermediate, float64:
    y_t = sum over the token's slots of w * (h_q . W2[e]^T) * s_h * s2, where a
    pseudo slot (e >= E) takes the shared W2 columns of its chunk.  shared =
    (h_vals [T, I_s], h_scale [T], gamma [T]) adds gamma_t * (h_t . Ws2^T) * s
    (the dense shared expert of the aux mode)."""
    from oracle import layer as L
    T, H, E, I, Is = cfg.T, cfg.H, cfg.E, cfg.I, cfg.I_s
    P = T * kt
    y = np.zeros((T, H))
    flat_ids = ids.reshape(-1)
    Wsh = L.shared_weights(host, cfg.fmt) if Is else None
    for e in range(E + (kt - cfg.topk)):
        slots = np.nonzero(srt < P)[0]
        slots = slots[flat_ids[srt[slots]] == e]
        if slots.size == 0:
            continue
        pairs = srt[slots]
        toks = pairs // kt
        if e < E:
            _, W2, _, s2 = L.expert_weights(host, cfg.fmt, e)
            hq = h_vals[slots]
        else:
            c = e - E
            wdt = min(I, Is - c * I)
            W2 = Wsh[1][:, c * I:c * I + wdt]
            s2 = Wsh[3]
            hq = h_vals[slots][:, :wdt]
        o = (hq @ W2.T) * h_scale[slots][:, None] * s2
        np.add.at(y, toks, w.reshape(-1)[pairs][:, None] * o)
    if shared is not None:
        hs_vals, hs_scale, gamma = shared
        y += gamma[:, None] * ((hs_vals @ Wsh[1].T) * hs_scale[:, None] * Wsh[3])
    return y


def adjacent_codes(a, b, sign_bit, mag_mask):
    """Codes one step apart (or equal) in a sign-magnitude format whose
    magnitudes are ordered like the codes (bf16 and e4m3fn both are)."""
    a, b = a.astype(np.int64), b.astype(np.int64)
    sa, sb = a & sign_bit, b & sign_bit
    ma, mb = a & mag_mask, b & mag_mask
    return np.where(sa == sb, np.abs(ma - mb) <= 1, (ma + mb) <= 1)


def compare_mx_h(got_q, got_s, h_exact, what):
    """A stage-1 MX-32 intermediate (e4m3 codes [n, K], e8m0 scales [n, K/32])
    against the oracle's exact h [n, K] (float64, before its bf16 rounding).

    A GPU value near a rounding boundary may land on the neighbouring code
    (fp32 against fp64 accumulation): such a code must be one step from the
    oracle's, or, for values far below their block's largest, within 2^-12 of
    that largest magnitude (the size of the fp32 accumulation error there).
    A block whose largest value crosses a power of two changes its scale by
    one, which requantises the block: such blocks are counted, not compared
    code by code.  Returns (values compared, values one code off, blocks,
    blocks with a scale one step off)."""
    import oracle
    rs, rq = oracle.mx_quantize(oracle.bf16_bits_to_f64(oracle.round_to_bf16_bits(h_exact)).astype(np.float32))
    same = got_s == rs
    assert (np.abs(got_s.astype(int) - rs.astype(int)) <= 1).all(), f"{what}: an MX block scale moved by more than one"
    cmp = np.repeat(same, 32, axis=1)
    diff = (got_q != rq) & cmp
    gv, rv = oracle.mx_dequantize(got_s, got_q), oracle.mx_dequantize(rs, rq)
    blk_max = np.repeat(np.abs(rv).reshape(rv.shape[0], -1, 32).max(axis=2), 32, axis=1)
    ok = adjacent_codes(got_q, rq, 0x80, 0x7F) | (np.abs(gv - rv) <= 2.0 ** -12 * blk_max)
    assert ok[diff].all(), f"{what}: {int((diff & ~ok).sum())} codes differ by more than one step"
    return int(cmp.sum()), int(diff.sum()), int(same.size), int((~same).sum())
