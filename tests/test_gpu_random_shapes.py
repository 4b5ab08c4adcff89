"""Randomised small shapes (hypothesis, derandomised so every run draws the same cases): the quantizers
bit-exact and the GEMMs within tolerance against the oracle, over shapes, strides, scale modes and output
types that the hand-written cases do not list.
"""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import fp8_fine_grained_amax_amd as fg
import oracle
from fp8_fine_grained_amax_amd import workloads as wl
from tests.gpu_util import TOL_BF16, TOL_F32, bf16_bits_to_f64, bits, device, normwise, np_u8, to_dev

pytestmark = pytest.mark.gpu

SETTINGS = settings(max_examples=25, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.function_scoped_fixture, HealthCheck.too_slow])


def _x(seed, rows, cols, ld, std=1.0, outliers=0):
    rng = np.random.default_rng(seed)
    full = wl.normal_bf16(rng, (rows, ld), std, outlier_channels=min(outliers, ld), outlier_scale=30.0)
    return full, to_dev(full)[:, :cols]


@SETTINGS
@given(rows=st.integers(1, 300), groups=st.integers(1, 5), pad=st.sampled_from([0, 8, 64]),
       pow2=st.booleans(), seed=st.integers(0, 2 ** 31 - 1))
def test_random_quantize_along_cols(rows, groups, pad, pow2, seed):
    device()
    cols = 128 * groups
    full, x = _x(seed, rows, cols, cols + pad, outliers=3)
    q, s = fg.fg_quantize_act_1x128(x, pow2=pow2)
    torch.cuda.synchronize()
    q_o, s_o = oracle.quantize_act_1x128(np.ascontiguousarray(bits(full)[:, :cols]), 0, pow2)
    assert np.array_equal(np_u8(q), q_o) and np.array_equal(s.cpu().numpy().view(np.uint32), s_o.view(np.uint32))


@SETTINGS
@given(row_tiles=st.integers(1, 3), cols8=st.integers(1, 40), pow2=st.booleans(), seed=st.integers(0, 2 ** 31 - 1))
def test_random_quantize_along_rows(row_tiles, cols8, pow2, seed):
    device()
    rows, cols = 128 * row_tiles, 8 * cols8
    full, x = _x(seed, rows, cols, cols, outliers=2)
    q, s = fg.fg_quantize_act_1x128(x, axis=fg.FG_ALONG_ROWS, pow2=pow2)
    torch.cuda.synchronize()
    q_o, s_o = oracle.quantize_act_1x128(bits(full), 1, pow2)
    assert np.array_equal(np_u8(q), q_o) and np.array_equal(s.cpu().numpy().view(np.uint32), s_o.view(np.uint32))


@SETTINGS
@given(M=st.integers(1, 520), N=st.integers(1, 520), kb=st.integers(1, 4), pow2=st.booleans(), bf16=st.booleans(),
       seed=st.integers(0, 2 ** 31 - 1))
def test_random_fprop(M, N, kb, pow2, bf16, seed):
    device()
    K = 128 * kb
    rng = np.random.default_rng(seed)
    x = wl.normal_bf16(rng, (M, K), 1.0, outlier_channels=2, outlier_scale=20.0)
    w = wl.normal_bf16(rng, (N, K), 0.02)
    xq, sx = fg.fg_quantize_act_1x128(to_dev(x), pow2=pow2)
    wq, sw = fg.fg_quantize_w_128x128(to_dev(w), pow2=pow2)
    y = fg.fg_fp8_gemm_fprop(xq, sx, wq, sw, out_dtype=torch.bfloat16 if bf16 else torch.float32, pow2=pow2)
    torch.cuda.synchronize()
    xq_o, sx_o = oracle.quantize_act_1x128(bits(x), 0, pow2)
    wq_o, sw_o = oracle.quantize_w_128x128(bits(w), pow2)
    prom, _ = oracle.gemm_fprop(xq_o, sx_o, wq_o, sw_o, out_bf16=bf16, want_exact=False)
    if bf16:
        assert normwise(bf16_bits_to_f64(bits(y).reshape(-1)), bf16_bits_to_f64(prom.reshape(-1))) <= TOL_BF16
    else:
        assert normwise(y.cpu().numpy(), prom) <= TOL_F32


@SETTINGS
@given(mt=st.integers(1, 3), N=st.integers(1, 300), K4=st.integers(1, 80), pow2=st.booleans(),
       seed=st.integers(0, 2 ** 31 - 1))
def test_random_wgrad(mt, N, K4, pow2, seed):
    device()
    M, K = 128 * mt, 4 * K4                        # M tokens (contraction), dW [N][K]
    rng = np.random.default_rng(seed)
    dy = wl.normal_bf16(rng, (M, N), 1e-3)
    x = wl.normal_bf16(rng, (M, K), 1.0)
    # the token-dim quantizer reads rows of 16 B: pad both operands' columns to multiples of 8, quantize,
    # and hand Wgrad the first N and K transposed rows
    def padded(t, c):
        out = torch.zeros((M, (c + 7) // 8 * 8), dtype=torch.bfloat16)
        out[:, :c] = t
        return out
    dyp, xp = padded(dy, N), padded(x, K)
    dytq, sdyt = fg.fg_quantize_act_1x128(to_dev(dyp), axis=fg.FG_ALONG_ROWS, pow2=pow2)
    xtq, sxt = fg.fg_quantize_act_1x128(to_dev(xp), axis=fg.FG_ALONG_ROWS, pow2=pow2)
    dw = fg.fg_fp8_gemm_wgrad(dytq[:N].contiguous(), sdyt[:, :N].contiguous(), xtq[:K].contiguous(),
                              sxt[:, :K].contiguous(), pow2=pow2)
    torch.cuda.synchronize()
    dytq_o, sdyt_o = oracle.quantize_act_1x128(bits(dyp), 1, pow2)
    xtq_o, sxt_o = oracle.quantize_act_1x128(bits(xp), 1, pow2)
    c = np.ascontiguousarray
    prom, _ = oracle.gemm_wgrad(c(dytq_o[:N]), c(sdyt_o[:, :N]), c(xtq_o[:K]), c(sxt_o[:, :K]), want_exact=False)
    assert normwise(dw.cpu().numpy(), prom) <= TOL_F32
