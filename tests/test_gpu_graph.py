"""The fine-grained FP8 Linear step captured in a HIP graph: every replay must reproduce the eager step
bit for bit (all kernels are deterministic), with the program's own eager work and synchronisations
between replays. The step is the benchmark's: X and dY quantized in both 1x128 tilings, W in 128x128
blocks, Fprop (BF16 out), Dgrad and Wgrad (FP32 out), at a shape of several tiles with ragged edges.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_amax_amd as fg
from fp8_fine_grained_amax_amd import workloads as wl
from tests.gpu_util import device, to_dev

pytestmark = pytest.mark.gpu


def _step(x, w, dy, pow2):
    xq, sx, xtq, sxt = fg.fg_quantize_act_1x128_both(x, pow2=pow2)
    wq, sw = fg.fg_quantize_w_128x128(w, pow2=pow2)
    y = fg.fg_fp8_gemm_fprop(xq, sx, wq, sw, pow2=pow2)
    dyq, sdy, dytq, sdyt = fg.fg_quantize_act_1x128_both(dy, pow2=pow2)
    dx = fg.fg_fp8_gemm_dgrad(dyq, sdy, wq, sw, pow2=pow2)
    dw = fg.fg_fp8_gemm_wgrad(dytq, sdyt, xtq, sxt, pow2=pow2)
    return [xq, sx, xtq, sxt, wq, sw, y, dyq, sdy, dytq, sdyt, dx, dw]


@pytest.mark.parametrize("pow2", [False, True])
def test_step_graph_replays_match_eager(pow2):
    device()
    rng = np.random.default_rng(71)
    M, N, K = 640, 896, 1152
    x = to_dev(wl.normal_bf16(rng, (M, K), 1.0, outlier_channels=8, outlier_scale=20.0))
    w = to_dev(wl.normal_bf16(rng, (N, K), 0.02))
    dy = to_dev(wl.normal_bf16(rng, (M, N), 1e-3))
    eager = [t.clone() for t in _step(x, w, dy, pow2)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    _step(x, w, dy, pow2)                                # warm the launch path outside the capture
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        outs = _step(x, w, dy, pow2)
    for replay in range(4):
        for t in outs:
            t.fill_(0) if t.dtype != torch.uint8 else t.fill_(0x55)    # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {replay}: output {i} differs"
