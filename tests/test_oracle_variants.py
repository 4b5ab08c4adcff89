"""Pins for the oracle's variants of the tiles: per-tensor scaling (the contrast baseline) and token tiles
re-quantized from cached 1x128 FP8 tiles. CPU only.

Per-tensor scaling maps a whole tensor's max-abs onto the largest E4M3 value ("5 Ways You can get More
Deepseek While Spending Less", the passage on the usual FP8 recipe and its outlier sensitivity); delayed
scaling takes that max-abs from a history of earlier iterations ("Three Fast Methods To Study Deepseek",
the passage on delayed quantization). Pinned against library routines (numpy max, fp32 division, torch's
E4M3 cast after clipping to +-448), against the tile quantizers on tensors that are one tile, and against
closed forms of the scale and of saturation.

Re-quantization reads activations cached as FP8 1x128 tiles for the backward pass (the Figure 6
passage) and forms the token tiles Wgrad needs. Pinned against the composition through library routines
(torch's E4M3 decode and bf16 cast, then the already pinned token-dim quantizer), and against the
arithmetic fact that power-of-2 scales add no rounding in E4M3's normal range.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_fine_grained_amax_amd import workloads as wl

FLT_MIN = np.float32(2.0 ** -126)


def _act(rows, cols, seed, std=1.0, outliers=0, outlier_scale=30.0):
    rng = np.random.default_rng(seed)
    return wl.bf16_bits(wl.normal_bf16(rng, (rows, cols), std, outlier_channels=outliers, outlier_scale=outlier_scale))


def _library_per_tensor(xbits, amax, pow2):
    """The definition through library routines: s = fp32 amax/448 (pow2: next power of two up), fp32
    division, clip to +-448, torch's float8_e4m3fn cast."""
    x = oracle.bf16_bits_to_f32(xbits)
    s = np.float32(1.0) if amax == 0 else np.float32(np.float32(amax) / np.float32(448.0))
    s = max(s, FLT_MIN)
    if pow2:
        m, e = np.frexp(s)
        s = s if m == 0.5 else np.float32(np.ldexp(1.0, e))
    qv = np.clip((x / s).astype(np.float32), -448.0, 448.0).astype(np.float32)
    return torch.from_numpy(qv).to(torch.float8_e4m3fn).view(torch.uint8).numpy(), np.float32(s)


def test_amax_matches_numpy():
    xb = _act(77, 384, 1, outliers=2)
    assert oracle.amax_bf16(xb) == np.abs(oracle.bf16_bits_to_f32(xb)).max()
    assert oracle.amax_bf16(np.zeros((3, 128), np.uint16)) == 0.0


@pytest.mark.parametrize("pow2", [False, True])
def test_current_scaling_matches_library_route(pow2):
    xb = _act(93, 512, 2, outliers=3)
    amax = oracle.amax_bf16(xb)
    q, s = oracle.quantize_per_tensor(xb, [amax], pow2, layout=0)
    q2, s2 = _library_per_tensor(xb, amax, pow2)
    assert s.shape == (4, 93) and (s == s2).all()
    assert np.array_equal(q, q2)
    if not pow2:
        assert (q & 0x7F).max() == 0x7E        # the tensor's max-abs lands on 448


@pytest.mark.parametrize("pow2", [False, True])
def test_one_tile_tensor_equals_tile_quantizers(pow2):
    """A tensor that is a single 1x128 tile (or a single 128x128 block) has the same scale and codes under
    per-tensor scaling as under the fine-grained quantizers."""
    xb = _act(1, 128, 3)
    q, s = oracle.quantize_per_tensor(xb, [oracle.amax_bf16(xb)], pow2, layout=0)
    qt, st = oracle.quantize_act_1x128(xb, 0, pow2)
    assert np.array_equal(q, qt) and np.array_equal(s, st)
    wb = _act(128, 128, 4, std=0.02)
    q, s = oracle.quantize_per_tensor(wb, [oracle.amax_bf16(wb)], pow2, layout=1)
    qw, sw = oracle.quantize_w_128x128(wb, pow2)
    assert np.array_equal(q, qw) and np.array_equal(s, sw)


@pytest.mark.parametrize("pow2", [False, True])
def test_delayed_scaling_saturates_above_history(pow2):
    xb = _act(64, 256, 5)
    x = oracle.bf16_bits_to_f32(xb)
    amax = oracle.amax_bf16(xb)
    hist = [0.25 * amax, 0.5 * amax, -0.4 * amax]          # |entries|; the largest is half the current
    q, s = oracle.quantize_per_tensor(xb, hist, pow2, layout=0)
    a = float(np.float32(0.5 * amax))
    q2, s2 = _library_per_tensor(xb, a, pow2)
    assert (s == s2).all() and np.array_equal(q, q2)
    big = np.abs(x / s2) > 448.0
    assert big.any() and ((q[big] & 0x7F) == 0x7E).all()
    assert np.array_equal(q[big] >> 7, (x[big] < 0).astype(np.uint8))
    # a history above the current max-abs: nothing saturates, codes as with that larger scale
    q3, s3 = oracle.quantize_per_tensor(xb, [4.0 * amax], pow2, layout=0)
    q4, s4 = _library_per_tensor(xb, float(np.float32(4.0 * amax)), pow2)
    assert (s3 == s4).all() and np.array_equal(q3, q4) and (q3 & 0x7F).max() < 0x7E


def test_history_reading_round_up_to_bf16_and_empty():
    xb = _act(4, 128, 6)
    # 1 + 2^-10 is between bf16 numbers: the next bf16 number up, 1 + 2^-7, is used
    _, s = oracle.quantize_per_tensor(xb, [1.0 + 2.0 ** -10], False)
    assert s[0, 0] == np.float32(np.float32(1.0 + 2.0 ** -7) / np.float32(448.0))
    # exactly representable: used as is
    _, s = oracle.quantize_per_tensor(xb, [3.0], False)
    assert s[0, 0] == np.float32(np.float32(3.0) / np.float32(448.0))
    # empty history: max-abs 0, scale 1, codes are enc(x) with saturation
    q, s = oracle.quantize_per_tensor(xb, [], False)
    assert (s == 1.0).all()
    assert np.array_equal(q, _library_per_tensor(xb, 0.0, False)[0])
    # beyond the largest finite bf16: capped there
    _, s = oracle.quantize_per_tensor(xb, [3.4e38], False)
    assert s[0, 0] == np.float32(np.float32(np.ldexp(255.0 / 128.0, 127)) / np.float32(448.0))


def test_scale_layouts():
    xb = _act(300, 384, 7)
    _, s0 = oracle.quantize_per_tensor(xb, [2.0], False, layout=0)
    _, s1 = oracle.quantize_per_tensor(xb, [2.0], False, layout=1)
    assert s0.shape == (3, 300) and s1.shape == (3, 3)
    assert (s0 == s0[0, 0]).all() and (s1 == s0[0, 0]).all()


def test_outliers_hurt_per_tensor_more_than_tiles():
    """The pages' point against per-tensor scaling: one outlier channel stretches the tensor's scale, and
    the ordinary values lose precision; 1x128 tiles confine the damage to the tiles holding the outlier.
    E4M3's 17 binades (subnormals included) absorb moderate outliers, so the loss shows once the outlier
    pushes ordinary values into the subnormal range: measured at a x10^4 outlier channel."""
    rng = np.random.default_rng(8)
    xf = rng.standard_normal((256, 1024), dtype=np.float32)
    xf[:, 17] *= np.float32(1e4)
    xb = wl.bf16_bits(wl.to_bf16(xf))
    x = oracle.bf16_bits_to_f32(xb).astype(np.float64)
    qt, st = oracle.quantize_act_1x128(xb, 0, False)
    qp, sp = oracle.quantize_per_tensor(xb, [oracle.amax_bf16(xb)], False)
    deq_t = oracle.e4m3_decode(qt) * np.repeat(st.T, 128, axis=1)
    deq_p = oracle.e4m3_decode(qp) * np.repeat(sp.T, 128, axis=1)
    ordinary = np.ones(1024, bool)
    ordinary[:128] = False                                 # channels outside the outlier's tiles
    nsr = lambda d: np.sqrt(((d - x)[:, ordinary] ** 2).mean() / (x[:, ordinary] ** 2).mean())
    flushed = lambda q: ((q[:, ordinary] & 0x7F) == 0).mean()
    assert nsr(deq_t) < 0.03 and nsr(deq_p) > 1.5 * nsr(deq_t)
    assert flushed(qt) < 1e-4 and flushed(qp) > 0.01


# ------------------------------------------------------------------------------------------------
# Token tiles re-quantized from cached 1x128 FP8 tiles
# ------------------------------------------------------------------------------------------------

def _library_dequant_bf16(q, s):
    """bf16 bits of bf16(RN_f32(decoded code * row scale)) through torch's E4M3 decode and bf16 cast."""
    d = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float32)
    sc = torch.from_numpy(np.repeat(s.T, 128, axis=1))
    return (d * sc).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("pow2_in,pow2_out", [(False, False), (True, True), (False, True)])
def test_requantize_is_token_quantization_of_the_cached_activation(pow2_in, pow2_out):
    xb = _act(256, 384, 11, outliers=3)
    q, s = oracle.quantize_act_1x128(xb, 0, pow2_in)
    qt, st = oracle.requantize_1x128_to_tokens(q, s, pow2_out)
    q2, s2 = oracle.quantize_act_1x128(_library_dequant_bf16(q, s), 1, pow2_out)
    assert qt.shape == (384, 256) and st.shape == (2, 384)
    assert np.array_equal(qt, q2) and np.array_equal(st, s2)


def test_requantize_pow2_adds_no_rounding_in_the_normal_range():
    """With power-of-2 scales the cached values are E4M3 numbers times 2^k; dividing by another power of
    two keeps their 4 significant bits, so a re-quantized value equals the cached one wherever it stays
    in E4M3's normal range."""
    xb = _act(512, 256, 12, outliers=2)
    q, s = oracle.quantize_act_1x128(xb, 0, True)
    qt, st = oracle.requantize_1x128_to_tokens(q, s, True)
    cached = oracle.e4m3_decode(q) * np.repeat(s.T, 128, axis=1)                  # [rows, cols]
    requant = (oracle.e4m3_decode(qt) * np.repeat(st.T, 128, axis=1)).T          # back to [rows, cols]
    normal = np.abs(cached) / np.repeat(st, 128, axis=0) >= 2.0 ** -6
    assert normal.mean() > 0.95
    assert np.array_equal(requant[normal], cached[normal])


def test_requantize_fp32_scales_round_twice():
    """With fp32 scales the re-quantized token tiles carry both roundings: their error against the original
    activations exceeds that of token tiles quantized from the activations directly. With power-of-2
    scales every orientation of the tiles rounds each value to the same 4 significant bits (normal range),
    so the re-quantized, the direct token and the row tiles agree."""
    xb = _act(512, 512, 13)
    x = oracle.bf16_bits_to_f32(xb).astype(np.float64)
    rms = lambda d: np.sqrt(((d - x) ** 2).mean() / (x ** 2).mean())
    deq_t = lambda qq, ss: (oracle.e4m3_decode(qq) * np.repeat(ss.T, 128, axis=1)).T
    errs = {}
    for pow2 in (False, True):
        q, s = oracle.quantize_act_1x128(xb, 0, pow2)
        qt, st = oracle.requantize_1x128_to_tokens(q, s, pow2)
        qd, sd = oracle.quantize_act_1x128(xb, 1, pow2)
        errs[pow2] = (rms(deq_t(qt, st)), rms(deq_t(qd, sd)))
    assert errs[False][0] > 1.2 * errs[False][1]
    assert abs(errs[True][0] - errs[True][1]) < 1e-9
