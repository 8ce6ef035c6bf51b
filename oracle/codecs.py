"""Number formats used by the layer, decoded and encoded from their definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Formats:

* bfloat16 -- the top 16 bits of an IEEE binary32; rounding is to nearest,
  ties to even (RNE).
* e4m3fn (OCP 8-bit float, "FN" flavour): sign, 4 exponent bits with bias 7,
  3 mantissa bits; exponent field 0 encodes subnormals 2^-6 * M/8; the code
  S.1111.111 is NaN; there is no infinity; the largest finite value is 448.
  AITER PR 6106 (Technical Details) treats the "fnuz" flavour as a separate
  path; this layer uses the OCP one.
* e8m0 -- an unsigned power-of-two scale 2^(b-127); b = 255 is NaN.
* MX-32 (OCP Microscaling v1.0): blocks of 32 consecutive elements along the
  reduction axis share one e8m0 scale.  AITER PR 6106 (Technical Details)
  states that the MXFP8 GEMM uses a K block of 32 and requires K % 32 == 0.
  Shared exponent: floor(log2(amax)) - 8 (8 = the largest exponent of e4m3),
  clamped to [-127, 127]; elements are v * 2^-exponent rounded RNE to e4m3 and
  saturated to +-448.  An all-zero block gets scale byte 0 and zero codes.
* e2m1 (OCP MX FP4): sign, 2 exponent bits with bias 1, 1 mantissa bit;
  exponent field 0 encodes the subnormals 0 and 0.5; no infinity or NaN; the
  largest value is 6.  Two elements per byte, element 2i in the low nibble of
  byte i (the order the gfx950 block-scaled MFMA reads them in).  The pages
  deploy MXFP4 expert weights (vLLM PR 65207, Purpose, commit 3: Quark MXFP4
  checkpoints; SGLang PR 27057, Modifications, item 1) without restating the
  format; MXFP4 = MX-32 blocks of e2m1 elements with an e8m0 scale.
* per-row e4m3 (used for the stage-2 input in the a8w8 layer): one fp32 scale
  per row, s = amax / 448, codes = e4m3_rne_sat(v * (448 / amax)), both
  products in fp32; an all-zero row gets s = 1 and zero codes.  The pages name
  per-token activation scales (AITER PR 6106, Technical Details) but do not
  say how the intermediate is quantised; this is the plainest reading.
"""

import numpy as np

E4M3_MAX = 448.0


def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16_bits(x):
    """Round real values (float64, treated as exact) to bfloat16, RNE.

    Returns uint16 bit patterns.  Inputs are finite.  The rounding is done on
    the exact value: 8 significant bits for normal numbers, a fixed quantum of
    2^-133 in the subnormal range, overflow to infinity past the largest finite
    bfloat16.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, e = np.frexp(ax)                     # ax = m * 2^e, m in [0.5, 1)
    q_exp = np.maximum(e - 8, -133)         # quantum exponent
    r = np.rint(np.ldexp(ax, -q_exp))       # exact scaling, then ties-to-even
    val = np.ldexp(r, q_exp)
    bf16_max = float(np.frombuffer(np.uint32(0x7F7F0000).tobytes(), np.float32)[0])
    val = np.where(val > bf16_max, np.inf, val)
    bits = (val.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    sign = np.signbit(x).astype(np.uint16) << np.uint16(15)
    return bits | sign


def _e4m3_closed_form(c):
    c = np.asarray(c, dtype=np.int64)
    s = c >> 7
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    sub = np.ldexp(m / 8.0, -6)
    v = np.where(e == 0, sub, normal)
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return np.where(s == 1, -v, v)


# the 256 values of the closed form, looked up by code
_E4M3_TABLE = _e4m3_closed_form(np.arange(256))


def e4m3_decode(codes):
    """e4m3fn codes (uint8) -> float64, by the closed form of the format
    (sign, 4-bit exponent with bias 7, 3-bit mantissa, subnormals at E = 0,
    S.1111.111 = NaN), tabulated once for all 256 codes."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode_rne_sat(x):
    """Real values -> nearest e4m3fn code, ties to even, saturating at +-448.

    Inputs are finite and treated as exact (float32 values pass through float64
    without change).  Normal range: 3 mantissa bits, quantum 2^(floor(log2|x|)-3);
    below 2^-6 the quantum is the subnormal step 2^-9.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, e = np.frexp(ax)
    flog2 = e - 1                                   # floor(log2 ax) for ax > 0
    q_exp = np.where(ax < 2.0 ** -6, -9, flog2 - 3)
    val = np.ldexp(np.rint(np.ldexp(ax, -q_exp)), q_exp)
    val = np.minimum(val, E4M3_MAX)                 # saturate (also covers ax >= 448)
    # value -> code
    _, ev = np.frexp(val)
    ev = ev - 1
    is_norm = val >= 2.0 ** -6
    mant = np.where(is_norm, (np.ldexp(val, -np.where(is_norm, ev, 0)) - 1.0) * 8.0, 0.0)
    code_norm = ((ev + 7) << 3) + mant.astype(np.int64)
    code_sub = np.ldexp(val, 9).astype(np.int64)
    code = np.where(is_norm, code_norm, code_sub)
    code = code | (np.signbit(x).astype(np.int64) << 7)
    return code.astype(np.uint8)


def e2m1_decode(codes):
    """e2m1 codes (0..15) -> float64 by the closed form: (-1)^S * 2^(E-1) *
    (1 + M/2) for E > 0, (-1)^S * M/2 for E = 0."""
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    v = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, e - 1))
    return np.where(s == 1, -v, v)


def e2m1_unpack(packed):
    """Bytes [..., K/2] holding two e2m1 codes each -> codes [..., K]
    (element 2i from the low nibble of byte i, 2i+1 from the high one)."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0x0F
    out[..., 1::2] = b >> 4
    return out


def mx4_dequantize(scales, packed):
    """MXFP4: (e8m0 scale bytes [..., K/32], packed e2m1 [..., K/2]) -> float64 [..., K]."""
    vals = e2m1_decode(e2m1_unpack(packed))
    K = vals.shape[-1]
    blocks = vals.reshape(vals.shape[:-1] + (K // 32, 32))
    return (blocks * e8m0_decode(scales)[..., None]).reshape(vals.shape)


def e8m0_decode(b):
    """e8m0 scale bytes -> float64 2^(b-127); 255 is NaN."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)


def _floor_log2(a):
    """floor(log2 a) for a > 0 (exact, from the binary exponent)."""
    _, e = np.frexp(np.asarray(a, dtype=np.float64))
    return e - 1


def mx_quantize(v):
    """MX-32 e4m3 quantisation along the last axis (OCP MX v1.0 rule).

    v: float32 array [..., K] with K % 32 == 0.
    Returns (scale bytes uint8 [..., K/32], codes uint8 [..., K]).
    The per-block exponent is exact; the element scaling v * 2^-X is done in
    float32, then rounded to e4m3 (RNE, saturating).
    """
    v = np.asarray(v, dtype=np.float32)
    K = v.shape[-1]
    assert K % 32 == 0
    blocks = v.reshape(v.shape[:-1] + (K // 32, 32))
    amax = np.max(np.abs(blocks), axis=-1)
    X = np.where(amax > 0, _floor_log2(np.where(amax > 0, amax, 1.0)) - 8, -127)
    X = np.clip(X, -127, 127)
    scaled = np.ldexp(blocks, (-X)[..., None].astype(np.int32))   # float32, exact power-of-two scaling
    codes = e4m3_encode_rne_sat(scaled.astype(np.float32))
    return (X + 127).astype(np.uint8), codes.reshape(v.shape)


def mx_dequantize(scales, codes):
    """MX-32 e4m3: (scale bytes [..., K/32], codes [..., K]) -> float64 [..., K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    K = codes.shape[-1]
    vals = e4m3_decode(codes).reshape(codes.shape[:-1] + (K // 32, 32))
    return (vals * e8m0_decode(scales)[..., None]).reshape(codes.shape)


def row_quantize_e4m3(v):
    """Per-row e4m3 quantisation with one fp32 scale per row.

    v: float32 [rows, K].  Returns (scale float32 [rows], codes uint8 [rows, K])
    with s = amax / 448 and codes = e4m3_rne_sat(v * (448 / amax)), every
    arithmetic step in float32; all-zero rows give s = 1 and zero codes.
    """
    v = np.asarray(v, dtype=np.float32)
    amax = np.max(np.abs(v), axis=-1)
    nz = amax > 0
    safe = np.where(nz, amax, np.float32(1))
    inv = np.float32(E4M3_MAX) / safe
    s = safe / np.float32(E4M3_MAX)
    scaled = (v * inv[:, None]).astype(np.float32)
    codes = e4m3_encode_rne_sat(scaled)
    codes = np.where(nz[:, None], codes, np.uint8(0)).astype(np.uint8)
    s = np.where(nz, s, np.float32(1)).astype(np.float32)
    return s, codes
