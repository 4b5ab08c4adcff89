"""GPU parity of the Fprop whose output is quantized on chip (fg_fp8_gemm_fprop_quant).

Its codes and 1x128 scales must be bit-identical to quantizing the BF16 output of fg_fp8_gemm_fprop on
the same operands. Checked three ways on every case:
  * against the oracle's 1x128 quantizer applied to that BF16 output (the independent check);
  * against the GPU quantizer fg_quantize_act_1x128 applied to it;
  * with the reference output computed under both workgroup shapes (the fused path always uses the
    256x256 shape; the result of the unfused GEMM must not depend on the shape).
The BF16 output itself is checked against the oracle's promoted GEMM (normwise, <= 1e-2) on the small
cases; the unfused GEMM's own parity is covered by the GEMM tests.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_amax_amd as fg
import oracle
from fp8_fine_grained_amax_amd import workloads as wl
from tests.gpu_util import TOL_BF16, bf16_bits_to_f64, bits, device, normwise, np_u8, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [(1, 128, 128), (130, 128, 256), (300, 512, 384), (200, 640, 256), (1000, 768, 512), (256, 2304, 1024)]
MODES = [(False, False), (True, True), (False, True), (True, False)]   # (operand scales, output scales)


def _operands(x, w, pow2):
    xq, sx = fg.fg_quantize_act_1x128(to_dev(x), pow2=pow2)
    wq, sw = fg.fg_quantize_w_128x128(to_dev(w), pow2=pow2)
    return xq, sx, wq, sw


def _unfused(ops, pow2, tile, monkeypatch):
    monkeypatch.setenv("FG_GEMM_TILE", tile)
    y = fg.fg_fp8_gemm_fprop(*ops, out_dtype=torch.bfloat16, pow2=pow2)
    torch.cuda.synchronize()
    monkeypatch.delenv("FG_GEMM_TILE", raising=False)
    return y


def _check(x, w, pow2, out_pow2, monkeypatch, oracle_gemm=False):
    ops = _operands(x, w, pow2)
    yq, sy = fg.fg_fp8_gemm_fprop_quant(*ops, pow2=pow2, out_pow2=out_pow2)
    torch.cuda.synchronize()
    yq_n, sy_n = np_u8(yq), sy.cpu().numpy()
    ys = [_unfused(ops, pow2, t, monkeypatch) for t in ("256x256", "256x192")]
    assert np.array_equal(bits(ys[0]), bits(ys[1])), "unfused BF16 output depends on the workgroup shape"
    yb = bits(ys[0])
    q_o, s_o = oracle.quantize_act_1x128(yb, 0, out_pow2)
    assert np.array_equal(sy_n.view(np.uint32), s_o.view(np.uint32)), "scales differ from the oracle's"
    bad = np.argwhere(yq_n != q_o)
    assert bad.size == 0, f"{len(bad)} codes differ from the oracle's, first at {bad[:4].tolist()}"
    q_g, s_g = fg.fg_quantize_act_1x128(ys[0], pow2=out_pow2)
    torch.cuda.synchronize()
    assert np.array_equal(np_u8(q_g), yq_n) and np.array_equal(s_g.cpu().numpy().view(np.uint32), sy_n.view(np.uint32))
    if oracle_gemm:
        xq_o, sx_o = oracle.quantize_act_1x128(bits(x), 0, pow2)
        wq_o, sw_o = oracle.quantize_w_128x128(bits(w), pow2)
        prom_bf16, _ = oracle.gemm_fprop(xq_o, sx_o, wq_o, sw_o, out_bf16=True, want_exact=False)
        assert normwise(bf16_bits_to_f64(yb), bf16_bits_to_f64(prom_bf16)) <= TOL_BF16
    return yq_n, sy_n


@pytest.mark.parametrize("pow2,out_pow2", MODES)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_fused_matches_quantized_output(M, N, K, pow2, out_pow2, monkeypatch):
    device()
    rng = np.random.default_rng(M * 7 + N * 3 + K + 2 * pow2 + out_pow2)
    x = wl.normal_bf16(rng, (M, K), 1.0, outlier_channels=min(4, K // 64), outlier_scale=20.0)
    w = wl.normal_bf16(rng, (N, K), 0.02)
    _check(x, w, pow2, out_pow2, monkeypatch, oracle_gemm=(pow2 == out_pow2))


@pytest.mark.parametrize("out_pow2", [False, True])
def test_fused_tiny_and_zero_rows(out_pow2, monkeypatch):
    """Rows whose output scale falls below 2^-100 (the quotient's shifted form) next to ordinary rows in
    the same 16-row MFMA tile, rows whose output is near the bottom of the normal range, and all-zero rows
    (scale 1, codes 0)."""
    device()
    M, N, K = 300, 384, 256
    rng = np.random.default_rng(77)
    xf = rng.standard_normal((M, K), dtype=np.float32)
    xf[0::3] *= np.float32(2.0 ** -60)
    xf[1::7] *= np.float32(2.0 ** -75)
    xf[5::11] = 0.0
    x = wl.to_bf16(xf)
    w = wl.to_bf16(rng.standard_normal((N, K), dtype=np.float32) * np.float32(2.0 ** -40))
    yq, sy = _check(x, w, False, out_pow2, monkeypatch)
    assert (sy < 2.0 ** -100).any() and (sy > 2.0 ** -100).any()
    assert np.all(sy[:, 5::11] == 1.0) and np.all(yq[5::11] == 0)


def test_fused_k0_writes_zero_codes_unit_scales():
    device()
    M, N = 200, 256
    xq = torch.empty((M, 0), dtype=torch.uint8, device="cuda")
    wq = torch.empty((N, 0), dtype=torch.uint8, device="cuda")
    sx = torch.empty((0, M), dtype=torch.float32, device="cuda")
    sw = torch.empty((N // 128, 0), dtype=torch.float32, device="cuda")
    yq = torch.full((M, N), 0x55, dtype=torch.uint8, device="cuda")
    sy = torch.full((N // 128, M), 3.0, dtype=torch.float32, device="cuda")
    fg.fg_fp8_gemm_fprop_quant(xq, sx, wq, sw, yq=yq, sy=sy)
    torch.cuda.synchronize()
    assert np.all(np_u8(yq) == 0) and np.all(sy.cpu().numpy() == 1.0)


@pytest.mark.parametrize("pow2", [False, True])
def test_fused_dsv3_mlp_full(pow2, monkeypatch):
    """The dense MLP shape X [4096, 7168] . W [18432, 7168]^T: all 75.5 M codes and 0.59 M scales."""
    device()
    x, w = wl.dsv3_fprop()
    ops = _operands(x, w, pow2)
    yq, sy = fg.fg_fp8_gemm_fprop_quant(*ops, pow2=pow2, out_pow2=pow2)
    monkeypatch.delenv("FG_GEMM_TILE", raising=False)
    y = fg.fg_fp8_gemm_fprop(*ops, out_dtype=torch.bfloat16, pow2=pow2)
    torch.cuda.synchronize()
    q_o, s_o = oracle.quantize_act_1x128(bits(y), 0, pow2)
    assert np.array_equal(sy.cpu().numpy().view(np.uint32), s_o.view(np.uint32))
    assert np.array_equal(np_u8(yq), q_o)
