"""Pins of the oracle's number-format codecs against things other than themselves:
the OCP E4M3 landmark table, torch's float8/bfloat16 casts (library routines),
brute-force nearest-code search, and crafted MX-32 blocks."""

import os

import numpy as np
import pytest
import torch

import oracle
from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e4m3_values():
    return oracle.e4m3_decode(np.arange(256, dtype=np.uint8))


def test_e4m3_landmarks_from_spec_table():
    with open(os.path.join(GOLDEN, "e4m3_landmarks.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for code, val in rows:
        got = oracle.e4m3_decode(np.uint8(int(code, 16)))
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val), (code, got, val)
            assert np.signbit(got) == val.startswith("-")


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = _e4m3_values()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def _brute_nearest(x):
    """Nearest e4m3 code by exhaustive search; ties to the even code; saturating."""
    vals = _e4m3_values()[:0x7F]  # non-negative finite codes 0..0x7E
    a = abs(float(x))
    if a >= 448:
        best = 0x7E
    else:
        d = np.abs(vals - a)
        m = d.min()
        cands = np.nonzero(d == m)[0]
        best = int(cands[0]) if len(cands) == 1 else int([c for c in cands if c % 2 == 0][0])
    return best | (0x80 if np.signbit(x) else 0)


def test_e4m3_encode_matches_brute_force():
    rng = np.random.default_rng(1)
    vals = _e4m3_values()[:0x7F]
    mids = (vals[:-1] + vals[1:]) / 2
    xs = np.concatenate([
        rng.normal(0, 100, 3000), rng.normal(0, 0.01, 2000), rng.uniform(-600, 600, 1000),
        mids, -mids, vals, -vals, [0.0, -0.0, 447.99, 448.0, 449.0, 463.99, 464.0, 1e6, 2.0 ** -10, 2.0 ** -10 * 3],
    ]).astype(np.float32)
    got = oracle.e4m3_encode_rne_sat(xs)
    ref = np.array([_brute_nearest(x) for x in xs], dtype=np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(xs[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(2)
    xs = np.concatenate([rng.normal(0, 50, 20000), rng.normal(0, 1e-2, 20000)]).astype(np.float32)
    xs = xs[np.abs(xs) <= 448]
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode_rne_sat(xs), ref)


def test_bf16_round_matches_torch_for_fp32():
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.normal(0, 1, 50000), rng.normal(0, 1e-30, 1000), rng.normal(0, 1e30, 1000)]).astype(np.float32)
    # exact ties: the low half is 0x8000
    ties = (rng.integers(0, 2 ** 31, 2000, dtype=np.uint32) & 0xFFFF0000) | 0x8000
    xs = np.concatenate([xs, ties.view(np.float32)[np.isfinite(ties.view(np.float32))]])
    ref = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_to_bf16_bits(xs.astype(np.float64))
    assert np.array_equal(got, ref)
    assert np.array_equal(oracle.bf16_bits_to_f64(got), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_bf16_round_is_single_rounding_of_the_exact_value():
    # 1 + 2^-8 is the midpoint between bf16 1.0 and 1 + 2^-7; a hair above it
    # must round up even though float32 would first round it onto the midpoint.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert oracle.bf16_bits_to_f64(oracle.round_to_bf16_bits(np.array([x])))[0] == 1.0 + 2.0 ** -7
    assert oracle.bf16_bits_to_f64(oracle.round_to_bf16_bits(np.array([1.0 + 2.0 ** -8])))[0] == 1.0


def test_e8m0():
    got = oracle.e8m0_decode(np.array([0, 1, 126, 127, 128, 254, 255], dtype=np.uint8))
    assert got[0] == 2.0 ** -127 and got[1] == 2.0 ** -126 and got[2] == 0.5
    assert got[3] == 1.0 and got[4] == 2.0 and got[5] == 2.0 ** 127 and np.isnan(got[6])


def test_mx_crafted_blocks():
    blk = np.zeros((4, 32), np.float32)
    blk[0, :] = np.linspace(-1, 1, 32)       # amax = 1 -> X = -8, 1.0 * 2^8 = 256 -> code 0x78
    blk[1, :] = 0.0                           # zero block -> byte 0, zero codes
    blk[2, 0] = 500.0                         # amax in [448, 512): X = 0, saturates to 448
    blk[2, 1] = -3.0
    blk[3, :] = 2.0 ** -130                   # sub-normal amax: exponent clamps at -127
    sc, q = oracle.mx_quantize(blk.reshape(1, 128))
    sc, q = sc.reshape(4), q.reshape(4, 32)
    assert sc[0] == 127 - 8 and q[0, -1] == 0x78 and q[0, 0] == 0xF8
    assert sc[1] == 0 and not q[1].any()
    assert sc[2] == 127 and q[2, 0] == 0x7E and oracle.e4m3_decode(q[2, 1]) == -3.0
    assert sc[3] == 0
    deq = oracle.mx_dequantize(sc.reshape(1, 4), q.reshape(1, 128)).reshape(4, 32)
    # element error <= half an e4m3 ulp (2^-4 relative) except the saturated one
    rel = np.abs(deq[0] - blk[0]) / np.maximum(np.abs(blk[0]), 2.0 ** -9 * 2.0 ** -8)
    assert np.all(rel <= 2.0 ** -4 + 1e-12)


def test_mx_roundtrip_random_blocks():
    rng = np.random.default_rng(4)
    v = (rng.normal(0, 1, (64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))).astype(np.float32)
    sc, q = oracle.mx_quantize(v)
    deq = oracle.mx_dequantize(sc, q)
    blocks = v.reshape(64, 8, 32)
    amax = np.abs(blocks).max(-1)
    # shared exponent puts the block amax in [256, 512) before quantisation
    X = sc.astype(np.int64) - 127
    assert np.all(amax * np.exp2(-X.astype(float)) >= 256) and np.all(amax * np.exp2(-X.astype(float)) < 512)
    # error bound: half ulp of e4m3 at the element's binade, or saturation to 448 * 2^X
    err = np.abs(deq.reshape(64, 8, 32) - blocks)
    bound = np.maximum(np.abs(blocks) * 2.0 ** -4, np.exp2(X - 9 - 1.0)[..., None]) + \
        np.maximum(0, amax - 448 * np.exp2(X))[..., None]
    assert np.all(err <= bound * (1 + 1e-9))


def test_row_quantize():
    v = np.zeros((3, 64), np.float32)
    v[1, :8] = [448, -448, 1, 2, 3, 0.5, 100, -7]
    v[2] = np.linspace(-2, 3, 64).astype(np.float32)
    s, q = oracle.row_quantize_e4m3(v)
    assert s[0] == 1.0 and not q[0].any()
    assert s[1] == 1.0 and np.array_equal(oracle.e4m3_decode(q[1, :8]), [448, -448, 1, 2, 3, 0.5, 96, -7])
    assert s[2] == np.float32(3.0) / np.float32(448)
    assert q[2, -1] == 0x7E


def _golden_e2m1():
    rows = []
    for line in open(os.path.join(GOLDEN, "e2m1_values.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            code, val = line.split()
            rows.append((int(code, 2), float(val)))
    return rows


def test_e2m1_decode_matches_the_ocp_table():
    rows = _golden_e2m1()
    assert [c for c, _ in rows] == list(range(16))
    got = oracle.e2m1_decode(np.arange(16))
    want = np.array([v for _, v in rows])
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))  # -0.0 for code 1000


def test_e2m1_unpack_nibble_order_and_mx4_scales():
    # byte 0x21: element 0 = low nibble 0001 (0.5), element 1 = high nibble 0010 (1.0)
    assert oracle.e2m1_unpack(np.array([0x21, 0xF7], np.uint8)).tolist() == [1, 2, 7, 15]
    packed = np.tile(np.array([0x21], np.uint8), (2, 16))  # two rows of 32 elements
    scales = np.array([[127], [130]], np.uint8)              # 2^0 and 2^3
    v = oracle.mx4_dequantize(scales, packed)
    assert v.shape == (2, 32)
    assert np.array_equal(v[0], np.tile([0.5, 1.0], 16))
    assert np.array_equal(v[1], np.tile([4.0, 8.0], 16))
