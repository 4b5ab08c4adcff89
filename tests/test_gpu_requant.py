"""GPU parity of token tiles re-quantized from cached 1x128 FP8 tiles (fg_requantize_1x128_to_tokens).

Codes and scales must equal the oracle's bit for bit: the cached codes' bf16 activations
bf16(RN_f32(code * row scale)), quantized along the tokens. Cases: several 128x128 tiles, every
combination of scale modes in and out, rows whose cached values are tiny (column scales below 2^-100)
or zero, and the full dense-MLP activation X [4096, 7168] in the launch configuration the benchmark
times. The extra rounding of the re-quantized tiles against tiles quantized straight from the bf16
activations is measured on the full-size X and printed.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_amax_amd as fg
import oracle
from fp8_fine_grained_amax_amd import workloads as wl
from tests.gpu_util import bits, device, np_u8, to_dev

pytestmark = pytest.mark.gpu

MODES = [(False, False), (True, True), (False, True), (True, False)]   # (cached tiles, token tiles)


def _check(xb_t, pow2_in, pow2_out):
    q, s = fg.fg_quantize_act_1x128(xb_t, pow2=pow2_in)
    qt, st = fg.fg_requantize_1x128_to_tokens(q, s, pow2=pow2_out)
    torch.cuda.synchronize()
    q_n, s_n = np_u8(q), s.cpu().numpy()
    qt_o, st_o = oracle.requantize_1x128_to_tokens(q_n, s_n, pow2_out)
    assert np.array_equal(st.cpu().numpy().view(np.uint32), st_o.view(np.uint32)), "scales differ from the oracle's"
    bad = np.argwhere(np_u8(qt) != qt_o)
    assert bad.size == 0, f"{len(bad)} codes differ from the oracle's, first at {bad[:4].tolist()}"
    return q_n, s_n, np_u8(qt), st.cpu().numpy()


@pytest.mark.parametrize("pow2_in,pow2_out", MODES)
@pytest.mark.parametrize("rows,cols", [(128, 128), (256, 384), (640, 1024)])
def test_requantize_exact(rows, cols, pow2_in, pow2_out):
    device()
    rng = np.random.default_rng(rows + cols + 2 * pow2_in + pow2_out)
    x = to_dev(wl.normal_bf16(rng, (rows, cols), 1.0, outlier_channels=min(4, cols // 64), outlier_scale=20.0))
    _check(x, pow2_in, pow2_out)


def test_requantize_tiny_and_zero():
    device()
    rng = np.random.default_rng(61)
    xf = rng.standard_normal((256, 256), dtype=np.float32)
    xf[:, 0:128] *= np.float32(1e-33)            # cached values far down: token scales below 2^-100
    xf[:, 200] = 0.0                             # an all-zero column: token scale 1, codes 0
    xf[7, :] = 0.0                               # an all-zero row: row scale 1
    x = to_dev(wl.to_bf16(xf))
    for pow2 in (False, True):
        _, _, qt, st = _check(x, pow2, pow2)
        assert (st[:, 200] == 1.0).all() and not qt[200].any()
    assert (st[:, :128] < 2.0 ** -100).all()


@pytest.mark.parametrize("pow2", [False, True])
def test_requantize_dsv3_activation_full(pow2):
    """X [4096, 7168] of the dense-MLP workload: all 29.4 M codes. Reports the error of the re-quantized
    token tiles and of token tiles quantized from the bf16 X, against X."""
    device()
    x, _ = wl.dsv3_fprop()
    xd = to_dev(x)
    _, _, qt, st = _check(xd, pow2, pow2)
    qd, sd = fg.fg_quantize_act_1x128(xd, axis=fg.FG_ALONG_ROWS, pow2=pow2)
    torch.cuda.synchronize()
    xf = oracle.bf16_bits_to_f32(bits(x)).astype(np.float64)[:1024]          # first 1024 tokens
    deq = lambda qq, ss: (oracle.e4m3_decode(qq[:, :1024]) * np.repeat(ss[:8].T, 128, axis=1)).T
    rms = lambda d: float(np.sqrt(((d - xf) ** 2).mean() / (xf ** 2).mean()))
    e_re, e_direct = rms(deq(qt, st)), rms(deq(np_u8(qd), sd.cpu().numpy()))
    print(f"\n[requant] {'pow2' if pow2 else 'fp32'} scales: re-quantized token tiles rms error {e_re:.4e}, "
          f"token tiles from bf16 {e_direct:.4e} (ratio {e_re / e_direct:.3f})")
    if pow2:
        assert abs(e_re - e_direct) < 1e-6
    else:
        assert e_re > 1.05 * e_direct
