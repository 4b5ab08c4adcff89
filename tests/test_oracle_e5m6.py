"""Pins for the oracle's E5M6 storage format (a reading of the customized format "5 Ways You can get More
Deepseek While Spending Less" names for cached activations with power-of-2 scaling factors). CPU only.

E5M6 is read as the E5 family's layout with a 6-bit fraction, which makes every code the top 12 bits of
an IEEE binary16 number: decode is pinned against numpy's float16 for all 4096 codes; encode against a
brute-force nearest search over the decoded table; the 1x128 quantizer against the composition of the
pinned pieces with numpy's scale arithmetic and an independent packing; dequantization against numpy's
rounding of bf16 values to 7 significant bits.
"""
import numpy as np
import pytest

import oracle
from fp8_fine_grained_amax_amd import workloads as wl

FLT_MIN = np.float32(2.0 ** -126)


def test_decode_is_binary16_top_bits_all_codes():
    codes = np.arange(4096, dtype=np.uint16)
    ref = (codes << 4).view(np.float16).astype(np.float64)
    got = oracle.e5m6_decode(codes)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.array_equal(np.isinf(got), np.isinf(ref))
    assert got[0x7BF] == 65024.0 and got[0x001] == 2.0 ** -20 and got[0x040] == 2.0 ** -14


def _brute_encode(v):
    table = oracle.e5m6_decode(np.arange(4096, dtype=np.uint16))
    pos = np.arange(0x7C0)                                  # finite non-negative codes, increasing values
    out = []
    for x in np.asarray(v, np.float64):
        a = min(abs(x), 65024.0)
        d = np.abs(table[pos] - a)
        best = np.flatnonzero(d == d.min())
        c = best[0] if len(best) == 1 else best[np.argmin(best & 1)]    # tie: the even code
        out.append(int(c) | (0x800 if np.signbit(x) else 0))
    return np.array(out, np.uint16)


def test_encode_brute_force():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(3000) * np.exp2(rng.uniform(-24, 17, 3000)),
                        [0.0, -0.0, 65024.0, 65023.0, 65535.0, 1e9, -1e9, 2.0 ** -20, 2.0 ** -21, 3 * 2.0 ** -21,
                         2.0 ** -14, -2.0 ** -14 * (1 - 2.0 ** -7)]]).astype(np.float32)
    assert np.array_equal(oracle.e5m6_encode(v), _brute_encode(v))


def test_encode_exact_midpoints_tie_to_even():
    table = oracle.e5m6_decode(np.arange(0x7C0, dtype=np.uint16))
    mids = ((table[:-1] + table[1:]) / 2).astype(np.float32)          # exact in float32 (<= 8 bits)
    got = oracle.e5m6_encode(mids)
    lo = np.arange(0x7BF, dtype=np.uint16)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1))


def _pack(codes):
    c = codes.astype(np.uint32).reshape(codes.shape[0], -1, 2)
    b = np.stack([c[..., 0] & 0xFF, (c[..., 0] >> 8) | ((c[..., 1] & 0xF) << 4), c[..., 1] >> 4], axis=-1)
    return b.reshape(codes.shape[0], -1).astype(np.uint8)


def test_quantize_matches_composition_of_pinned_pieces():
    rng = np.random.default_rng(2)
    xb = wl.bf16_bits(wl.normal_bf16(rng, (37, 384), 1.0, outlier_channels=3, outlier_scale=1e4))
    xb[5, :128] = 0                                         # zero tile: scale 1
    xb[6, 128:256] = wl.bf16_bits(wl.to_bf16(np.full((1, 128), 3e-38, np.float32)))   # scale clamps to FLT_MIN
    packed, s = oracle.quantize_e5m6_1x128(xb)
    x = oracle.bf16_bits_to_f32(xb)
    amax = np.abs(x.reshape(37, 3, 128)).max(axis=2)
    t = np.maximum((amax / np.float32(65024.0)).astype(np.float32), FLT_MIN)
    m, e = np.frexp(t)
    sc = np.where(m == 0.5, t, np.ldexp(np.float32(1.0), e)).astype(np.float32)
    sc = np.where(amax == 0, np.float32(1.0), sc)
    assert np.array_equal(s, sc.T)
    q = (x / np.repeat(sc, 128, axis=1)).astype(np.float32)
    codes = _brute_encode(q.reshape(-1)).reshape(q.shape)
    assert np.array_equal(packed, _pack(codes))
    assert np.array_equal(oracle.e5m6_unpack(packed), codes)
    assert s[1, 6] == FLT_MIN and s[0, 5] == 1.0


def test_dequantize_rounds_bf16_to_seven_significant_bits():
    """bf16 has 8 significant bits and E5M6 7: with exact power-of-2 scaling, storage rounds each value to
    7 significant bits (ties to even) wherever it stays normal in E5M6, and dequantization is exact."""
    rng = np.random.default_rng(3)
    xb = wl.bf16_bits(wl.normal_bf16(rng, (64, 512), 1.0))
    y = oracle.dequantize_e5m6_1x128(*oracle.quantize_e5m6_1x128(xb))
    u = xb.astype(np.uint32)
    r = ((u + ((u >> 1) & 1)) >> 1) << 1                           # drop the last bf16 fraction bit, RNE
    expected = r.astype(np.uint16)
    _, s = oracle.quantize_e5m6_1x128(xb)
    normal = np.abs(oracle.bf16_bits_to_f32(xb)) >= 2.0 ** -14 * np.repeat(s.T, 128, axis=1)
    assert normal.mean() > 0.99
    assert np.array_equal(y[normal], expected[normal])


def _golden(kind):
    path = __file__.rsplit("/", 1)[0] + "/golden/e5m6_worked_examples.txt"
    for line in open(path):
        if line.startswith(kind + " |"):
            yield [f.strip() for f in line.split("|")[1:]]


def test_golden_worked_codes():
    """Hand-derived codes (tests/golden/e5m6_worked_examples.txt): normal, subnormal, saturated values and
    exact ties to the even code, through both the encoder and the decoder."""
    rows = list(_golden("code"))
    assert len(rows) == 13
    vals = np.array([float(v) for v, _ in rows], np.float32)
    want = np.array([int(c, 16) for _, c in rows], np.uint16)
    assert np.array_equal(oracle.e5m6_encode(vals), want)
    dec = oracle.e5m6_decode(want)
    assert dec[0] == 1.0 and dec[1] == -3.0 and dec[2] == 0.099609375 and dec[3] == 65024.0


def test_golden_worked_tile():
    """A hand-derived 1x128 tile: its power-of-2 scale, its codes and their three-bytes-per-two packing."""
    (vals, scale, codes, packed), = list(_golden("tile"))
    x = np.zeros((1, 128), np.float32)
    v = [float(t) for t in vals.split()]
    x[0, :len(v)] = v
    xb = wl.bf16_bits(wl.to_bf16(x))
    p, s = oracle.quantize_e5m6_1x128(xb)
    assert s[0, 0] == np.float32(float(scale))
    c = [int(t, 16) for t in codes.split()]
    assert np.array_equal(oracle.e5m6_unpack(p)[0, :len(c)], np.array(c, np.uint16))
    b = [int(t, 16) for t in packed.split()]
    assert np.array_equal(p[0, :len(b)], np.array(b, np.uint8))
    assert np.array_equal(oracle.dequantize_e5m6_1x128(p, s)[0, :3], xb[0, :3])
