"""GPU parity of E5M6 storage (fg_quantize_e5m6_1x128 / fg_dequantize_e5m6_1x128) against the oracle, bit
for bit: packed codes, power-of-2 scales and the dequantized bf16 values. Cases: ragged rows, several
column groups, row strides wider than the row, zero tiles, tiles whose scale clamps to FLT_MIN, values in
E5M6's subnormal range next to the largest bf16 numbers, and the full dense-MLP activation
X [4096, 7168]. The storage error is compared with the FP8 1x128 tiles' on that X and printed.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_amax_amd as fg
import oracle
from fp8_fine_grained_amax_amd import workloads as wl
from tests.gpu_util import bits, device, np_u8, to_dev

pytestmark = pytest.mark.gpu


def _check(x_t):
    packed, s = fg.fg_quantize_e5m6_1x128(x_t)
    y = fg.fg_dequantize_e5m6_1x128(packed, s)
    torch.cuda.synchronize()
    xb = np.ascontiguousarray(bits(x_t))
    p_o, s_o = oracle.quantize_e5m6_1x128(xb)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_o.view(np.uint32)), "scales differ from the oracle's"
    bad = np.argwhere(np_u8(packed) != p_o)
    assert bad.size == 0, f"{len(bad)} packed bytes differ from the oracle's, first at {bad[:4].tolist()}"
    y_o = oracle.dequantize_e5m6_1x128(p_o, s_o)
    assert np.array_equal(bits(y), y_o), "dequantized values differ from the oracle's"
    return xb, s.cpu().numpy(), bits(y)


@pytest.mark.parametrize("rows,cols,ld", [(1, 128, 128), (45, 384, 392), (300, 1024, 1024)])
def test_e5m6_exact(rows, cols, ld):
    device()
    rng = np.random.default_rng(rows + cols)
    full = wl.normal_bf16(rng, (rows, ld), 1.0, outlier_channels=min(4, ld // 64), outlier_scale=1e3)
    _check(to_dev(full)[:, :cols])


def test_e5m6_edge_tiles():
    device()
    rng = np.random.default_rng(5)
    xf = rng.standard_normal((64, 512), dtype=np.float32)
    xf[3, :128] = 0.0                                      # zero tile: scale 1
    xf[4, 128:256] = np.float32(3e-38)                     # scale clamps to FLT_MIN
    xf[5, 256:384] *= np.float32(1e-30)                    # tiny tile
    xf[6, 384:] = np.float32(1e-6)                         # E5M6 subnormals next to ...
    xf[6, 400] = np.float32(3.3e38)                        # ... the largest bf16 numbers
    xf[7, 384] = np.float32(-0.0)
    _, s, _ = _check(to_dev(wl.to_bf16(xf)))
    assert s[0, 3] == 1.0 and s[1, 4] == np.float32(2.0 ** -126)


def test_e5m6_dsv3_activation_full():
    """X [4096, 7168]: all 44 M packed bytes; storage error against X beside the FP8 tiles'."""
    device()
    x, _ = wl.dsv3_fprop()
    xd = to_dev(x)
    xb, _, yb = _check(xd)
    q8, s8 = fg.fg_quantize_act_1x128(xd)
    torch.cuda.synchronize()
    xf = oracle.bf16_bits_to_f32(xb[:512]).astype(np.float64)
    e5 = oracle.bf16_bits_to_f32(yb[:512]).astype(np.float64)
    f8 = oracle.e4m3_decode(np_u8(q8)[:512]) * np.repeat(s8.cpu().numpy()[:, :512].T, 128, axis=1)
    rms = lambda d: float(np.sqrt(((d - xf) ** 2).mean() / (xf ** 2).mean()))
    print(f"\n[e5m6] rms storage error: E5M6 {rms(e5):.3e} (1.5 B/value), FP8 E4M3 {rms(f8):.3e} (1 B/value)")
    # 7 of bf16's 8 significant bits survive: the dropped bit costs at most one bf16 unit, 2^-7 relative
    nz = np.abs(xf) >= 1e-6                                   # far above the tiles' subnormal range here
    assert (np.abs(e5 - xf)[nz] <= 2.0 ** -7 * np.abs(xf)[nz]).all()
    assert rms(e5) < rms(f8) / 3
