"""Pins for the CPU oracle, against facts fixed outside the oracle itself.

Each test ties one oracle function to something independent of it: values the pages fix (golden fixtures
with their citations), hand-derived worked examples, closed forms, brute force over the decode table,
library routines (torch's float8_e4m3fn and bfloat16 casts, numpy float64 matmul) and invariants of the
method. CPU only.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_amax_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FLT_MIN = np.float32(2.0 ** -126)


def _f32_bits(v):
    return np.array(v, dtype=np.float32).view(np.uint32)


def _bits_f32(u):
    return np.array(u, dtype=np.uint32).view(np.float32)


# ------------------------------------------------------------------------------------------------
# E4M3 decode / encode
# ------------------------------------------------------------------------------------------------

def test_decode_golden_values():
    for line in open(os.path.join(GOLDEN, "e4m3_format.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code, val = line.split()
        got = oracle.e4m3_decode([int(code, 16)])[0]
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), (code, got, val)


def test_decode_matches_torch_float8_e4m3fn_all_codes():
    ours = oracle.e4m3_decode(np.arange(256))
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def _brute_force_encode(values):
    """Nearest finite E4M3 value by search over the decode table; ties -> even code (even mantissa);
    beyond 448 -> 448; sign of the input is kept (also for zero)."""
    table = oracle.e4m3_decode(np.arange(128))            # non-negative codes 0x00..0x7F
    finite = np.arange(127)                               # 0x7F is NaN
    mags = table[finite]
    a = np.abs(values.astype(np.float64))
    d = np.abs(a[:, None] - mags[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among equally near codes prefer the one with an even mantissa (code & 1 == 0)
    even = (finite % 2 == 0)[None, :]
    pick_even = cand & even
    has_even = pick_even.any(axis=1)
    idx = np.where(has_even, pick_even.argmax(axis=1), cand.argmax(axis=1))
    codes = finite[idx]
    codes = np.where(a >= 448.0, 0x7E, codes)
    return (codes | np.where(np.signbit(values), 0x80, 0)).astype(np.uint8)


def _structured_floats():
    """Every binary32 exponent that can matter (2^-140 .. 2^9) crossed with every pattern of the top 6
    mantissa bits and the low bits 0, 1, half, max: covers every E4M3 rounding boundary, tie and sticky
    case, for both signs."""
    vals = []
    for e in range(-140 + 127, 10 + 127):
        for top in range(64):
            for low in (0, 1, 1 << 16, (1 << 17) - 1, (1 << 17), (1 << 17) + 1):
                if e <= 0:
                    continue
                u = (e << 23) | (top << 17) | low
                vals.append(u)
    u = np.array(vals, dtype=np.uint32)
    sub = np.arange(0, 1 << 12, dtype=np.uint32) << 11         # binary32 subnormals
    u = np.concatenate([u, sub, [0]])
    f = _bits_f32(u)
    return np.concatenate([f, -f])


def _encode_many(vals):
    return np.array([oracle.e4m3_encode_scalar(v) for v in vals], dtype=np.uint8)


def test_encode_brute_force_structured():
    vals = _structured_floats()
    got = _encode_many(vals)
    exp = _brute_force_encode(vals)
    bad = np.nonzero(got != exp)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(exp[i])) for i in bad[:10]]


def test_encode_brute_force_random():
    rng = np.random.default_rng(11)
    # log-uniform magnitudes across the whole E4M3 range and beyond, random signs
    vals = (np.exp2(rng.uniform(-12, 10, 200_000)) * rng.choice([-1, 1], 200_000)).astype(np.float32)
    got = _encode_many(vals)
    exp = _brute_force_encode(vals)
    assert np.array_equal(got, exp)


def test_encode_midpoints_exact_ties():
    # Every midpoint between adjacent non-negative E4M3 values is a tie: it must go to the even code.
    mags = oracle.e4m3_decode(np.arange(127))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (mags[:-1] + mags[1:]) / 2)   # exactly representable
    got = _encode_many(mids)
    lo = np.arange(126)
    exp = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, exp.astype(np.uint8))


def test_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(12)
    vals = np.concatenate([
        (rng.uniform(-464, 464, 100_000)).astype(np.float32),
        (np.exp2(rng.uniform(-14, 8.8, 100_000)) * rng.choice([-1, 1], 100_000)).astype(np.float32),
    ])
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = _encode_many(vals)
    assert np.array_equal(got, ref)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(13)
    u = rng.integers(0, 0x7F000000, 200_000, dtype=np.uint32)
    # add exact ties and near-ties
    u = np.concatenate([u, (u & 0xFFFF0000) | 0x8000, (u & 0xFFFF0000) | 0x7FFF, (u & 0xFFFF0000) | 0x8001])
    f = _bits_f32(u)
    f = np.concatenate([f, -f])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16_scalar(v) for v in f], dtype=np.uint16)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------------------------------------
# Quantizers
# ------------------------------------------------------------------------------------------------

def _tile_bits(values):
    row = np.zeros(128, np.float32)
    row[: len(values)] = values
    bits = wl.bf16_bits(wl.to_bf16(row))
    assert np.array_equal(oracle.bf16_bits_to_f32(bits)[: len(values)], np.float32(values)), "not bf16-exact"
    return bits.reshape(1, 128)


def test_quantize_worked_examples():
    n = 0
    for line in open(os.path.join(GOLDEN, "quantize_worked_examples.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        mode, vals, scale, codes = [p.strip() for p in line.split("|")]
        vals = [float(v) for v in vals.split()]
        codes = [int(c, 16) for c in codes.split()]
        q, s = oracle.quantize_act_1x128(_tile_bits(vals), axis=0, pow2=(mode == "pow2"))
        assert s[0, 0] == np.float32(float(scale)), (line, s[0, 0])
        assert list(q[0, : len(codes)]) == codes, (line, [hex(c) for c in q[0, : len(codes)]])
        assert not q[0, len(codes):].any()
        n += 1
    assert n >= 8


def _rand_act(rows, cols, seed, scale=1.0, outliers=0):
    rng = np.random.default_rng(seed)
    return wl.bf16_bits(wl.normal_bf16(rng, (rows, cols), scale, outlier_channels=outliers, outlier_scale=30.0))


def _library_quantize_rows(xbits, pow2):
    """The definition through library routines: fp32 division by the scale, torch's E4M3 cast."""
    x = oracle.bf16_bits_to_f32(xbits)
    rows, cols = x.shape
    t = x.reshape(rows, cols // 128, 128)
    amax = np.abs(t).max(axis=2)
    s = (amax / np.float32(448.0)).astype(np.float32)
    s = np.where(s < FLT_MIN, FLT_MIN, s)
    if pow2:
        m, e = np.frexp(s)
        s = np.where(m == 0.5, s, np.ldexp(np.float32(1.0), e).astype(np.float32))
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    qv = (t / s[:, :, None]).astype(np.float32)
    q = torch.from_numpy(qv.reshape(rows, cols)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return q, s.T.copy()


@pytest.mark.parametrize("pow2", [False, True])
def test_quantize_rows_matches_library_route(pow2):
    xb = _rand_act(37, 512, 21, outliers=3)
    q, s = oracle.quantize_act_1x128(xb, axis=0, pow2=pow2)
    q2, s2 = _library_quantize_rows(xb, pow2)
    assert np.array_equal(s, s2)
    assert np.array_equal(q, q2)


@pytest.mark.parametrize("pow2", [False, True])
def test_quantize_axis1_is_transposed_axis0(pow2):
    xb = _rand_act(256, 72, 22)
    q1, s1 = oracle.quantize_act_1x128(xb, axis=1, pow2=pow2)
    q0, s0 = oracle.quantize_act_1x128(np.ascontiguousarray(xb.T), axis=0, pow2=pow2)
    assert q1.shape == (72, 256) and s1.shape == (2, 72)
    assert np.array_equal(q1, q0)
    assert np.array_equal(s1, s0)


@pytest.mark.parametrize("pow2", [False, True])
def test_quantize_weight_blocks_match_library_route(pow2):
    wb = _rand_act(256 + 40, 384, 23, scale=0.02)
    q, s = oracle.quantize_w_128x128(wb, pow2=pow2)
    w = oracle.bf16_bits_to_f32(wb)
    for bi in range(3):
        for bj in range(3):
            blk = w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            amax = np.float32(np.abs(blk).max())
            sc = np.float32(amax / np.float32(448.0))
            if pow2:
                m, e = np.frexp(sc)
                sc = sc if m == 0.5 else np.float32(np.ldexp(1.0, e))
            assert s[bi, bj] == sc
            ref = torch.from_numpy((blk / sc).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(q[bi * 128:bi * 128 + blk.shape[0], bj * 128:(bj + 1) * 128], ref)


def test_quantize_invariants_fp32_mode():
    xb = _rand_act(64, 1024, 24, outliers=4)
    q, s = oracle.quantize_act_1x128(xb, axis=0, pow2=False)
    mag = q & 0x7F
    # (i) every tile holds a code of magnitude 448
    assert (mag.reshape(64, 8, 128).max(axis=2) == 0x7E).all()
    # (iv) dequantization error at most half an E4M3 spacing at x/s, times s
    x = oracle.bf16_bits_to_f32(xb).astype(np.float64)
    deq = oracle.e4m3_decode(q) * np.repeat(s.T, 128, axis=1)
    v = np.abs(x) / np.repeat(s.T, 128, axis=1)
    spacing = np.where(v < 2 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(v, 2 ** -6))) - 3))
    assert (np.abs(deq - x) <= 0.5 * spacing * np.repeat(s.T, 128, axis=1) * (1 + 1e-6)).all()


def test_quantize_invariants_pow2_mode():
    xb = _rand_act(64, 1024, 25, outliers=4)
    q, s = oracle.quantize_act_1x128(xb, axis=0, pow2=True)
    m, _ = np.frexp(s)
    assert (m == 0.5).all()                                      # (ii) exact powers of two
    vmax = oracle.e4m3_decode(q & 0x7F).reshape(64, 8, 128).max(axis=2)
    assert ((vmax >= 224) & (vmax <= 448)).all()


def test_quantize_scaling_equivariance():
    # (iii) multiplying a tile by 2^j leaves the codes unchanged and multiplies the scale by 2^j
    xb = _rand_act(16, 256, 26)
    for pow2 in (False, True):
        q, s = oracle.quantize_act_1x128(xb, axis=0, pow2=pow2)
        for j in (-5, 3, 11):
            x2 = wl.bf16_bits(wl.to_bf16(oracle.bf16_bits_to_f32(xb) * np.float32(2.0 ** j)))
            q2, s2 = oracle.quantize_act_1x128(x2, axis=0, pow2=pow2)
            assert np.array_equal(q, q2)
            assert np.array_equal(s2, (s * np.float32(2.0 ** j)).astype(np.float32))


def test_quantize_zero_and_tiny_tiles():
    xb = np.zeros((3, 256), np.uint16)
    xb[1, 5] = 0x0001                       # smallest bf16 subnormal: 2^-133
    xb[2, 200] = 0x8080                     # -2^-126 (smallest normal, negative)
    q, s = oracle.quantize_act_1x128(xb, axis=0, pow2=False)
    assert s[0, 0] == 1.0 and s[1, 0] == 1.0 and not q[0].any()
    assert s[0, 1] == FLT_MIN               # amax/448 underflows below FLT_MIN -> FLT_MIN
    assert s[1, 2] == FLT_MIN and q[2, 200] == 0xB8   # -2^-126 / 2^-126 = -1
    assert q[1, 5] == 0x04                  # 2^-133 / 2^-126 = 2^-7 = 4 * 2^-9 -> subnormal code 4


def test_quantize_ragged_tiles():
    xb = _rand_act(5, 300, 27)
    q, s = oracle.quantize_act_1x128(xb, axis=0, pow2=False)
    assert s.shape == (3, 5)
    x = oracle.bf16_bits_to_f32(xb)
    assert np.array_equal(s[2], (np.abs(x[:, 256:]).max(axis=1) / np.float32(448)).astype(np.float32))


# ------------------------------------------------------------------------------------------------
# GEMMs
# ------------------------------------------------------------------------------------------------

def _rand_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, c & 0xF0, c).astype(np.uint8)   # no NaN codes


def _dequant_act(q, s):       # q [R, C], s [C/128, R]
    return oracle.e4m3_decode(q) * np.repeat(s.T.astype(np.float64), 128, axis=1)[:, : q.shape[1]]


def _dequant_w(q, s):         # q [N, K], s [N/128, K/128]
    full = np.repeat(np.repeat(s.astype(np.float64), 128, axis=0), 128, axis=1)
    return oracle.e4m3_decode(q) * full[: q.shape[0], : q.shape[1]]


@pytest.mark.parametrize("M,N,K", [(3, 5, 128), (8, 7, 256), (4, 130, 512)])
def test_fprop_exact_equals_float64_matmul(M, N, K):
    rng = np.random.default_rng(M * 1000 + N + K)
    xq, wq = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    sx = rng.uniform(0.01, 2, (K // 128, M)).astype(np.float32)
    sw = rng.uniform(0.01, 2, ((N + 127) // 128, K // 128)).astype(np.float32)
    prom, exact = oracle.gemm_fprop(xq, sx, wq, sw)
    ref = _dequant_act(xq, sx) @ _dequant_w(wq, sw).T
    assert np.allclose(exact, ref, rtol=1e-12, atol=1e-9 * np.abs(ref).max())
    # promoted vs exact: within the FP32 promotion bound (K/128 roundings of the running sum and the
    # block values, each at most 2^-24 relative to the magnitudes involved)
    terms = np.abs(_dequant_act(xq, sx)) @ np.abs(_dequant_w(wq, sw)).T
    assert (np.abs(prom - exact) <= 3 * (K // 128 + 1) * 2.0 ** -24 * terms + 1e-30).all()


def test_fprop_closed_forms():
    # all codes 1.0 with unit scales: every output equals K exactly
    K = 512
    xq = np.full((4, K), 0x38, np.uint8)
    wq = np.full((3, K), 0x38, np.uint8)
    prom, exact = oracle.gemm_fprop(xq, np.ones((4, 4), np.float32), wq, np.ones((1, 4), np.float32))
    assert (prom == K).all() and (exact == K).all()
    # one nonzero per block: the output is the sum of the selected products times their scales
    rng = np.random.default_rng(5)
    xq = np.zeros((1, K), np.uint8)
    wq = np.zeros((1, K), np.uint8)
    sx = np.array([[0.5], [2.0], [4.0], [0.25]], np.float32)
    sw = np.array([[1.0, 3.0, 0.5, 8.0]], np.float32)
    want = 0.0
    for b in range(4):
        k = b * 128 + int(rng.integers(0, 128))
        xq[0, k], wq[0, k] = 0x40 + b, 0xB8 - b       # 2*(1+b/8) and -(1 - ...) codes
        want += float(sx[b, 0] * sw[0, b]) * oracle.e4m3_decode([xq[0, k]])[0] * oracle.e4m3_decode([wq[0, k]])[0]
    prom, exact = oracle.gemm_fprop(xq, sx, wq, sw)
    assert exact[0, 0] == want


def test_promotion_worked_example():
    vals = {}
    for line in open(os.path.join(GOLDEN, "promotion_worked_example.txt")):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split("=")
            vals[k.strip()] = float(v)
    K = 384
    xq = np.zeros((1, K), np.uint8)
    wq = np.zeros((1, K), np.uint8)
    xq[0, 3], wq[0, 3] = 0x58, 0x58
    xq[0, 130], wq[0, 130] = 0x38, 0x38
    xq[0, 300], wq[0, 300] = 0x38, 0x38
    sx = np.array([[2.0 ** 16], [1.0], [1.0]], np.float32)
    sw = np.ones((1, 3), np.float32)
    prom, exact = oracle.gemm_fprop(xq, sx, wq, sw)
    assert prom[0, 0] == vals["promoted"]
    assert exact[0, 0] == vals["exact"]


def test_dgrad_exact_equals_float64_matmul():
    rng = np.random.default_rng(31)
    M, N, K = 6, 256, 200
    dyq, wq = _rand_codes(rng, (M, N)), _rand_codes(rng, (N, K))
    sdy = rng.uniform(0.01, 2, (N // 128, M)).astype(np.float32)
    sw = rng.uniform(0.01, 2, (N // 128, (K + 127) // 128)).astype(np.float32)
    prom, exact = oracle.gemm_dgrad(dyq, sdy, wq, sw)
    ref = _dequant_act(dyq, sdy) @ _dequant_w(wq, sw)
    assert np.allclose(exact, ref, rtol=1e-12, atol=1e-9 * np.abs(ref).max())
    assert np.allclose(prom, ref, rtol=1e-5, atol=1e-5 * np.abs(ref).max())


def test_wgrad_exact_equals_float64_matmul_and_accumulates():
    rng = np.random.default_rng(32)
    M, N, K = 256, 9, 130
    dyq, xq = _rand_codes(rng, (M, N)), _rand_codes(rng, (M, K))     # token-major codes
    sdy = rng.uniform(0.01, 2, (M // 128, N)).astype(np.float32)     # per (token block, channel)
    sx = rng.uniform(0.01, 2, (M // 128, K)).astype(np.float32)
    dytq, xtq = np.ascontiguousarray(dyq.T), np.ascontiguousarray(xq.T)
    prom, exact = oracle.gemm_wgrad(dytq, sdy, xtq, sx)
    dy = oracle.e4m3_decode(dyq) * np.repeat(sdy.astype(np.float64), 128, axis=0)
    x = oracle.e4m3_decode(xq) * np.repeat(sx.astype(np.float64), 128, axis=0)
    ref = dy.T @ x
    assert np.allclose(exact, ref, rtol=1e-12, atol=1e-9 * np.abs(ref).max())
    init = rng.standard_normal((N, K)).astype(np.float32)
    prom2, exact2 = oracle.gemm_wgrad(dytq, sdy, xtq, sx, dw_init=init)
    assert np.allclose(exact2, ref + init, rtol=1e-12, atol=1e-9 * np.abs(ref).max())
    assert np.allclose(prom2, ref + init, rtol=1e-5, atol=1e-5 * np.abs(ref).max())


def test_grouped_equals_per_group_fprop():
    rng = np.random.default_rng(33)
    K, N = 256, 136
    off = np.array([0, 5, 5, 40, 41], np.int32)          # includes an empty group
    G, T = 4, 41
    xq, wq = _rand_codes(rng, (T, K)), _rand_codes(rng, (G, N, K))
    sx = rng.uniform(0.01, 2, (K // 128, T)).astype(np.float32)
    sw = rng.uniform(0.01, 2, (G, 2, K // 128)).astype(np.float32)
    prom, exact = oracle.gemm_grouped(xq, sx, wq, sw, off, out_bf16=False)
    for g in range(G):
        a, b = off[g], off[g + 1]
        if a == b:
            continue
        ref = _dequant_act(xq[a:b], sx[:, a:b]) @ _dequant_w(wq[g], sw[g]).T
        assert np.allclose(exact[a:b], ref, rtol=1e-12, atol=1e-9 * np.abs(ref).max())


def test_points_match_full_and_bf16_output():
    rng = np.random.default_rng(34)
    M, N, K = 17, 140, 384
    xq, wq = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    sx = rng.uniform(0.01, 2, (3, M)).astype(np.float32)
    sw = rng.uniform(0.01, 2, (2, 3)).astype(np.float32)
    prom, exact = oracle.gemm_fprop(xq, sx, wq, sw)
    pts = rng.choice(M * N, 50, replace=False)
    p2, e2 = oracle.gemm_fprop(xq, sx, wq, sw, pts=pts)
    assert np.array_equal(p2, prom.reshape(-1)[pts]) and np.array_equal(e2, exact.reshape(-1)[pts])
    pb, _ = oracle.gemm_fprop(xq, sx, wq, sw, out_bf16=True, want_exact=False)
    ref = torch.from_numpy(prom).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(pb, ref)


# ------------------------------------------------------------------------------------------------
# Limited-precision accumulation (the pages' ~2% at K = 4096)
# ------------------------------------------------------------------------------------------------

def test_limited_accumulation_reproduces_pages_order_of_magnitude():
    facts = {}
    for line in open(os.path.join(GOLDEN, "limited_accumulation.txt")):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split("=")
            facts[k.strip()] = float(v)
    errs = {}
    for K in (4096, 16384):
        xb, wb = wl.accumulation_stress(K, M=8, N=8)
        xq, sx = oracle.quantize_act_1x128(wl.bf16_bits(xb), 0, False)
        wq, sw = oracle.quantize_w_128x128(wl.bf16_bits(wb), False)
        prom, exact = oracle.gemm_fprop(xq, sx, wq, sw)
        errs[(K, "promoted")] = np.max(np.abs(prom - exact) / np.abs(exact))
        for bits in (10, 11):
            lim = oracle.gemm_fprop_limited(xq, sx, wq, sw, chunk=32, bits=bits)
            errs[(K, bits)] = np.max(np.abs(lim - exact) / np.abs(exact))
    target = facts["max_rel_error_about"]
    assert int(facts["K"]) == 4096
    assert target / 4 <= errs[(4096, 10)] <= target * 4
    assert target / 4 <= errs[(4096, 11)] * 2 <= target * 4
    assert errs[(16384, 10)] > 2 * errs[(4096, 10)]           # grows with K
    assert errs[(4096, "promoted")] < 1e-6 and errs[(16384, "promoted")] < 1e-6


def test_encode_exhaustive_against_torch_cast():
    """Every non-negative float32 below 464 (1.14e9 bit patterns) and every 61st negative one: the oracle's
    encoder equals torch's float8_e4m3fn cast (a library routine; it rounds to nearest even and agrees with
    saturation up to 464, where it turns to NaN)."""
    top = int(np.array(464.0, np.float32).view(np.uint32))
    step = 1 << 26
    for start in range(0, top, step):
        u = np.arange(start, min(start + step, top), dtype=np.uint32)
        for bits_ in (u, (u[::61] | np.uint32(0x80000000))):
            v = bits_.view(np.float32)
            ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            got = oracle.e4m3_encode_many(v)
            bad = np.flatnonzero(got != ref)
            assert bad.size == 0, f"{bad.size} mismatches from {v[bad[0]]!r}: oracle {got[bad[0]]:#x}, torch {ref[bad[0]]:#x}"
