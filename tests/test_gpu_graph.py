"""The fine-grained FP8 Linear step captured in a HIP graph: every replay must reproduce the eager step
bit for bit (all kernels are deterministic), with the program's own eager work and synchronisations
between replays. The step is the benchmark's: X in both 1x128 tilings and W in 128x128 blocks from one
launch, dY in both tilings, Fprop (BF16 out), Dgrad and Wgrad (FP32 out), at a shape of several tiles with
ragged edges.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_amax_amd as fg
from fp8_fine_grained_amax_amd import workloads as wl
from tests.gpu_util import device, to_dev

pytestmark = pytest.mark.gpu


def _step(x, w, dy, pow2):
    xq, sx, xtq, sxt, wq, sw = fg.fg_quantize_fprop_operands(x, w, pow2=pow2)
    y = fg.fg_fp8_gemm_fprop(xq, sx, wq, sw, pow2=pow2)
    dyq, sdy, dytq, sdyt = fg.fg_quantize_act_1x128_both(dy, pow2=pow2)
    dx = fg.fg_fp8_gemm_dgrad(dyq, sdy, wq, sw, pow2=pow2)
    dw = fg.fg_fp8_gemm_wgrad(dytq, sdyt, xtq, sxt, pow2=pow2)
    return [xq, sx, xtq, sxt, wq, sw, y, dyq, sdy, dytq, sdyt, dx, dw]


@pytest.mark.parametrize("tile", ["auto", "256x288"])
@pytest.mark.parametrize("pow2", [False, True])
def test_step_graph_replays_match_eager(pow2, tile, monkeypatch):
    """"256x288" forces the Fprop onto its wide tile (the other GEMMs ignore that setting)."""
    if tile != "auto":
        monkeypatch.setenv("FG_GEMM_TILE", tile)
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


def test_every_entry_point_in_one_graph():
    """Every entry point of the library captured in one HIP graph (outputs allocated beforehand; the device
    max-abs is cleared and the accumulating Wgrad's dW reset by small fill and copy kernels inside the
    graph): three replays, with eager work between them, each equal to the eager sequence bit for bit."""
    device()
    dev = device()
    rng = np.random.default_rng(72)
    M, K, N = 256, 384, 256
    x = to_dev(wl.normal_bf16(rng, (M, K), 1.0, outlier_channels=4, outlier_scale=20.0))
    w = to_dev(wl.normal_bf16(rng, (N, K), 0.02))
    dy = to_dev(wl.normal_bf16(rng, (M, N), 1e-3))
    wg = to_dev(wl.normal_bf16(rng, (2 * N, K), 0.02))
    off_rows = torch.tensor([0, 100, M], dtype=torch.int32, device=dev)
    off_tok = torch.tensor([0, 128, M], dtype=torch.int32, device=dev)
    dw_init = torch.randn((N, K), dtype=torch.float32, device=dev)
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)
    o = {"xq": u8(M, K), "sx": f32(K // 128, M), "xtq": u8(K, M), "sxt": f32(M // 128, K),
         "xq2": u8(M, K), "sx2": f32(K // 128, M), "xtq2": u8(K, M), "sxt2": f32(M // 128, K),
         "xq3": u8(M, K), "sx3": f32(K // 128, M), "xtq3": u8(K, M), "sxt3": f32(M // 128, K),
         "wq3": u8(N, K), "sw3": f32(N // 128, K // 128),
         "wq": u8(N, K), "sw": f32(N // 128, K // 128), "wgq": u8(2, N, K), "swg": f32(2, N // 128, K // 128),
         "dyq": u8(M, N), "sdy": f32(N // 128, M), "dytq": u8(N, M), "sdyt": f32(M // 128, N),
         "rq": u8(K, M), "rs": f32(M // 128, K), "e5": u8(M, K * 3 // 2), "e5s": f32(K // 128, M),
         "e5y": torch.empty((M, K), dtype=torch.bfloat16, device=dev), "amax": f32(1),
         "pq": u8(M, K), "ps": f32(K // 128, M),
         "y": torch.empty((M, N), dtype=torch.bfloat16, device=dev), "yq": u8(M, N), "sy": f32(N // 128, M),
         "yl": f32(M, N), "dx": f32(M, K), "dw": f32(N, K), "dwa": f32(N, K),
         "gy": f32(M, N), "gdx": f32(M, K), "gdw": f32(2, N, K)}

    def run():
        fg.fg_quantize_act_1x128(x, q=o["xq"], scales=o["sx"])
        fg.fg_quantize_act_1x128(x, axis=fg.FG_ALONG_ROWS, q=o["xtq"], scales=o["sxt"])
        fg.fg_quantize_act_1x128_both(x, q_cols=o["xq2"], scales_cols=o["sx2"], q_rows=o["xtq2"], scales_rows=o["sxt2"])
        fg.fg_quantize_w_128x128(w, q=o["wq"], scales=o["sw"])
        fg.fg_quantize_fprop_operands(x, w, q_cols=o["xq3"], scales_cols=o["sx3"], q_rows=o["xtq3"],
                                      scales_rows=o["sxt3"], qw=o["wq3"], sw=o["sw3"])
        for g in range(2):
            fg.fg_quantize_w_128x128(wg[g * N:(g + 1) * N], q=o["wgq"][g], scales=o["swg"][g])
        fg.fg_quantize_act_1x128_both(dy, q_cols=o["dyq"], scales_cols=o["sdy"], q_rows=o["dytq"], scales_rows=o["sdyt"])
        fg.fg_requantize_1x128_to_tokens(o["xq"], o["sx"], q_out=o["rq"], s_out=o["rs"])
        fg.fg_quantize_e5m6_1x128(x, packed=o["e5"], scales=o["e5s"])
        fg.fg_dequantize_e5m6_1x128(o["e5"], o["e5s"], y=o["e5y"])
        o["amax"].zero_()
        fg.fg_amax_bf16(x, amax=o["amax"])
        fg.fg_quantize_per_tensor(x, o["amax"], q=o["pq"], scales=o["ps"])
        fg.fg_fp8_gemm_fprop(o["xq"], o["sx"], o["wq"], o["sw"], y=o["y"])
        fg.fg_fp8_gemm_fprop_quant(o["xq"], o["sx"], o["wq"], o["sw"], yq=o["yq"], sy=o["sy"])
        fg.fg_fp8_gemm_fprop_limited_accum(o["xq"], o["sx"], o["wq"], o["sw"], 10, y=o["yl"])
        fg.fg_fp8_gemm_dgrad(o["dyq"], o["sdy"], o["wq"], o["sw"], dx=o["dx"])
        fg.fg_fp8_gemm_wgrad(o["dytq"], o["sdyt"], o["xtq"], o["sxt"], dw=o["dw"])
        o["dwa"].copy_(dw_init)
        fg.fg_fp8_gemm_wgrad(o["dytq"], o["sdyt"], o["xtq"], o["sxt"], dw=o["dwa"], accumulate=True)
        fg.fg_fp8_grouped_gemm(o["xq"], o["sx"], o["wgq"], o["swg"], off_rows, out_dtype=torch.float32, y=o["gy"])
        fg.fg_fp8_grouped_gemm_dgrad(o["dyq"], o["sdy"], o["wgq"], o["swg"], off_rows, dx=o["gdx"])
        fg.fg_fp8_grouped_gemm_wgrad(o["dytq"], o["sdyt"], o["xtq"], o["sxt"], off_tok, dw=o["gdw"])

    run()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in o.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for replay in range(3):
        for t in o.values():
            t.view(torch.uint8).fill_(0x55)                    # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in o:
            assert torch.equal(o[k].view(torch.uint8), eager[k].view(torch.uint8)), f"replay {replay}: {k} differs"
