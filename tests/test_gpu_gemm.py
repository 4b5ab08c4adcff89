"""GPU parity: the HIP block-scaled FP8 GEMMs against the CPU oracle.

Gate: normwise max relative error against the oracle's per-128 FP32-promoted result, <= 1e-3 for FP32
outputs and <= 1e-2 for BF16 outputs (oracle rounded to BF16 too). The matrix core's summation inside
a 128-element block is hardware-defined, so results are not bit-identical; small shapes are compared in
full, the full-size workloads on sampled outputs computed one by one by the oracle, in the same launch
configuration the benchmark times: corners, the last row and column, random points, and one point in
every 64 x 64 output block (so every wave's tile of either workgroup shape is sampled). Every output
buffer starts filled with NaN and must come back entirely finite, so an element no kernel writes fails.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_amax_amd as fg
import oracle
from fp8_fine_grained_amax_amd import workloads as wl
from tests.gpu_util import (TOL_BF16, TOL_F32, assert_all_written, bf16_bits_to_f64, bits, device, nan_like_out,
                            normwise, np_u8, record_gemm_error, sample_points, stratified_points, to_dev)

pytestmark = pytest.mark.gpu


def _out_np(y, bf16):
    if bf16:
        return bits(y)
    return y.detach().cpu().numpy()


def _cmp(y_gpu, prom, bf16, tol_scale=1.0):
    if bf16:
        a, b = bf16_bits_to_f64(np.asarray(y_gpu).reshape(-1)), bf16_bits_to_f64(np.asarray(prom).reshape(-1))
        err = normwise(a, b)
        record_gemm_error("bf16", a, b)
        assert err <= TOL_BF16 * tol_scale, err
    else:
        a, b = np.asarray(y_gpu).reshape(-1), np.asarray(prom).reshape(-1)
        err = normwise(a, b)
        record_gemm_error("f32", a, b)
        assert err <= TOL_F32 * tol_scale, err
    return err


# The library picks one of two workgroup shapes per launch (256x192 with 12 waves, 256x256 with 8 waves)
# from the problem size, and for Fprop a third (256x288, 8 waves of 64x144); FG_GEMM_TILE forces one.
# Small shapes run under each, and under the automatic choice; the full-size cases run under the automatic
# choice, the configuration the benchmark times (256x288 for the dense-MLP Fprop).
TILES = ["auto", "256x192", "256x256"]
FPROP_TILES = TILES + ["256x288"]


@pytest.fixture
def tile(request, monkeypatch):
    if request.param == "auto":
        monkeypatch.delenv("FG_GEMM_TILE", raising=False)
    else:
        monkeypatch.setenv("FG_GEMM_TILE", request.param)
    return request.param


def _rand_act(rng, rows, cols, std=1.0):
    return wl.normal_bf16(rng, (rows, cols), std, outlier_channels=min(4, cols // 64), outlier_scale=20.0)


# ------------------------------------------------------------------------------------------------
# Fprop
# ------------------------------------------------------------------------------------------------

def _fprop_case(x, w, bf16, pow2=False, pts=None):
    xq, sx = fg.fg_quantize_act_1x128(to_dev(x), pow2=pow2)
    wq, sw = fg.fg_quantize_w_128x128(to_dev(w), pow2=pow2)
    y = nan_like_out((x.shape[0], w.shape[0]), torch.bfloat16 if bf16 else torch.float32)
    fg.fg_fp8_gemm_fprop(xq, sx, wq, sw, y=y, pow2=pow2)
    torch.cuda.synchronize()
    assert_all_written(y, "fprop")
    xq_n, sx_n, wq_n, sw_n = np_u8(xq), sx.cpu().numpy(), np_u8(wq), sw.cpu().numpy()
    # the codes the GEMM consumed are the oracle's codes (checked bit-exact in the quantizer tests);
    # re-derive them here from the oracle so the GEMM check does not trust the GPU quantizer
    xq_o, sx_o = oracle.quantize_act_1x128(bits(x), 0, pow2)
    wq_o, sw_o = oracle.quantize_w_128x128(bits(w), pow2)
    assert np.array_equal(xq_n, xq_o) and np.array_equal(wq_n, wq_o)
    assert np.array_equal(sx_n, sx_o) and np.array_equal(sw_n, sw_o)
    prom, exact = oracle.gemm_fprop(xq_o, sx_o, wq_o, sw_o, out_bf16=bf16, pts=pts)
    yo = _out_np(y, bf16).reshape(-1)
    yo = yo if pts is None else yo[pts]
    return _cmp(yo, prom, bf16), yo, exact


def test_fprop_tiny_config_fp32():
    device()
    x, w = wl.tiny_fprop()
    err, y, exact = _fprop_case(x, w, bf16=False)
    assert normwise(y, exact) <= TOL_F32


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (37, 130, 256), (256, 256, 128), (300, 520, 384),
                                   (513, 260, 640), (64, 1000, 1024), (1000, 64, 128), (300, 576, 384),
                                   (129, 1152, 512)])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("tile", FPROP_TILES, indirect=True)
def test_fprop_shapes(M, N, K, bf16, tile):
    device()
    rng = np.random.default_rng(M * 31 + N * 7 + K)
    _fprop_case(_rand_act(rng, M, K), wl.normal_bf16(rng, (N, K), 0.02), bf16)


@pytest.mark.parametrize("tile", FPROP_TILES, indirect=True)
def test_fprop_pow2_scales(tile):
    device()
    rng = np.random.default_rng(9)
    _fprop_case(_rand_act(rng, 200, 512), wl.normal_bf16(rng, (384, 512), 0.02), bf16=False, pow2=True)
    _fprop_case(_rand_act(rng, 300, 384), wl.normal_bf16(rng, (576, 384), 0.02), bf16=True, pow2=True)


@pytest.mark.parametrize("tile", FPROP_TILES, indirect=True)
def test_fprop_closed_form_all_ones(tile):
    # every code 1.0 (bf16 ones quantize to code 0x7E with scale 1/448): Y = K exactly
    device()
    M, N, K = 100, 300, 1024
    x = torch.ones((M, K), dtype=torch.bfloat16)
    w = torch.ones((N, K), dtype=torch.bfloat16)
    xq, sx = fg.fg_quantize_act_1x128(to_dev(x))
    wq, sw = fg.fg_quantize_w_128x128(to_dev(w))
    y = fg.fg_fp8_gemm_fprop(xq, sx, wq, sw, out_dtype=torch.float32).cpu().numpy()
    prom, _ = oracle.gemm_fprop(np_u8(xq), sx.cpu().numpy(), np_u8(wq), sw.cpu().numpy())
    assert np.array_equal(y, prom)
    assert np.allclose(y, K, rtol=1e-6)


@pytest.mark.parametrize("tile", FPROP_TILES, indirect=True)
def test_fprop_zero_k_writes_zeros(tile):
    device()
    y = torch.full((5, 7), 3.0, device=device())
    xq = torch.empty((5, 0), dtype=torch.uint8, device=device())
    wq = torch.empty((7, 0), dtype=torch.uint8, device=device())
    s = torch.empty((0,), dtype=torch.float32, device=device())
    fg.fg_fp8_gemm_fprop(xq, s, wq, s, y=y)
    assert torch.count_nonzero(y).item() == 0


@pytest.fixture(scope="module")
def dsv3():
    device()
    x, w = wl.dsv3_fprop()
    dy = wl.dsv3_backward_dy()
    return x, w, dy


@pytest.mark.parametrize("pow2", [False, True])
def test_fprop_dsv3_full_size_sampled(dsv3, pow2):
    x, w, _ = dsv3
    M, K = x.shape
    N = w.shape[0]
    pts = stratified_points(M, N, 3000, seed=11)
    err, y, exact = _fprop_case(x, w, bf16=True, pow2=pow2, pts=pts)
    assert normwise(bf16_bits_to_f64(y), exact) <= TOL_BF16


@pytest.mark.parametrize("M,N,bf16", [(8960, 16704, True), (4096, 18432, False), (16384, 8192, True)])
@pytest.mark.parametrize("pow2", [False, True])
def test_fprop_output_past_cache_size(M, N, bf16, pow2):
    """Outputs of 256 MiB or more are stored past the caches (a separate instantiation of each kernel):
    299 MB of BF16 and 302 MB of FP32 on 256x288 tiles, 268 MB of BF16 on 256x256 tiles, each tile the
    library's own choice on 256 compute units. K = 256 keeps the oracle's sampled check cheap; every 64x64 output block
    is sampled and the NaN-filled output must come back entirely written."""
    device()
    rng = np.random.default_rng(M + N + (7 if bf16 else 3))
    K = 256
    pts = stratified_points(M, N, 2000, seed=17)
    _fprop_case(_rand_act(rng, M, K), wl.normal_bf16(rng, (N, K), 0.02), bf16=bf16, pow2=pow2, pts=pts)


def test_fprop_deterministic(dsv3):
    x, w, _ = dsv3
    xq, sx = fg.fg_quantize_act_1x128(to_dev(x))
    wq, sw = fg.fg_quantize_w_128x128(to_dev(w))
    y1 = fg.fg_fp8_gemm_fprop(xq, sx, wq, sw)
    y2 = fg.fg_fp8_gemm_fprop(xq, sx, wq, sw)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# ------------------------------------------------------------------------------------------------
# Dgrad
# ------------------------------------------------------------------------------------------------

def _dgrad_case(dy, w, bf16, pts=None, pow2=False):
    dyq, sdy = fg.fg_quantize_act_1x128(to_dev(dy), pow2=pow2)
    wq, sw = fg.fg_quantize_w_128x128(to_dev(w), pow2=pow2)
    dx = nan_like_out((dy.shape[0], w.shape[1]), torch.bfloat16 if bf16 else torch.float32)
    fg.fg_fp8_gemm_dgrad(dyq, sdy, wq, sw, dx=dx, pow2=pow2)
    torch.cuda.synchronize()
    assert_all_written(dx, "dgrad")
    dyq_o, sdy_o = oracle.quantize_act_1x128(bits(dy), 0, pow2)
    wq_o, sw_o = oracle.quantize_w_128x128(bits(w), pow2)
    assert np.array_equal(np_u8(dyq), dyq_o) and np.array_equal(np_u8(wq), wq_o)
    prom, exact = oracle.gemm_dgrad(dyq_o, sdy_o, wq_o, sw_o, out_bf16=bf16, pts=pts)
    yo = _out_np(dx, bf16).reshape(-1)
    yo = yo if pts is None else yo[pts]
    return _cmp(yo, prom, bf16), yo, exact


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (37, 256, 128), (300, 384, 640), (256, 128, 256), (100, 512, 384),
                                   (300, 256, 896), (129, 384, 1152)])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("tile", TILES, indirect=True)
def test_dgrad_shapes(M, N, K, bf16, pow2, tile):
    device()
    rng = np.random.default_rng(M * 13 + N * 5 + K)
    _dgrad_case(_rand_act(rng, M, N, 1e-3), wl.normal_bf16(rng, (N, K), 0.02), bf16, pow2=pow2)


@pytest.mark.parametrize("pow2", [False, True])
def test_dgrad_dsv3_full_size_sampled(dsv3, pow2):
    x, w, dy = dsv3
    M, N = dy.shape
    K = w.shape[1]
    pts = stratified_points(M, K, 2000, seed=12)
    err, y, exact = _dgrad_case(dy, w, bf16=False, pts=pts, pow2=pow2)
    assert normwise(y, exact) <= TOL_F32


# ------------------------------------------------------------------------------------------------
# Wgrad
# ------------------------------------------------------------------------------------------------

def _wgrad_case(dy, x, pts=None, init=None, pow2=False):
    dytq, sdyt = fg.fg_quantize_act_1x128(to_dev(dy), axis=fg.FG_ALONG_ROWS, pow2=pow2)
    xtq, sxt = fg.fg_quantize_act_1x128(to_dev(x), axis=fg.FG_ALONG_ROWS, pow2=pow2)
    N, K = dy.shape[1], x.shape[1]
    if init is not None:
        dw = to_dev(torch.from_numpy(init))
        dw = fg.fg_fp8_gemm_wgrad(dytq, sdyt, xtq, sxt, dw=dw, accumulate=True, pow2=pow2)
    else:
        dw = nan_like_out((N, K), torch.float32)
        fg.fg_fp8_gemm_wgrad(dytq, sdyt, xtq, sxt, dw=dw, pow2=pow2)
    torch.cuda.synchronize()
    assert_all_written(dw, "wgrad")
    dytq_o, sdyt_o = oracle.quantize_act_1x128(bits(dy), 1, pow2)
    xtq_o, sxt_o = oracle.quantize_act_1x128(bits(x), 1, pow2)
    assert np.array_equal(np_u8(dytq), dytq_o) and np.array_equal(np_u8(xtq), xtq_o)
    init_sel = None if init is None else (init.reshape(-1) if pts is None else init.reshape(-1)[pts])
    prom, exact = oracle.gemm_wgrad(dytq_o, sdyt_o, xtq_o, sxt_o, dw_init=init_sel, pts=pts)
    yo = dw.cpu().numpy().reshape(-1)
    yo = yo if pts is None else yo[pts]
    return _cmp(yo, prom, False), yo, exact


@pytest.mark.parametrize("M,N,K", [(128, 8, 8), (128, 40, 264), (256, 296, 384), (384, 256, 128), (512, 136, 72),
                                   (384, 520, 640)])
@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("tile", TILES, indirect=True)
def test_wgrad_shapes(M, N, K, pow2, tile):
    device()
    rng = np.random.default_rng(M + N * 3 + K * 11)
    _wgrad_case(_rand_act(rng, M, N, 1e-3), _rand_act(rng, M, K), pow2=pow2)


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("tile", TILES, indirect=True)
def test_wgrad_accumulate(pow2, tile):
    device()
    rng = np.random.default_rng(5)
    M, N, K = 256, 200, 136
    init = rng.standard_normal((N, K)).astype(np.float32) * 1e-3
    _wgrad_case(_rand_act(rng, M, N, 1e-3), _rand_act(rng, M, K), init=init, pow2=pow2)


@pytest.mark.parametrize("pow2", [False, True])
def test_wgrad_dsv3_full_size_sampled(dsv3, pow2):
    x, w, dy = dsv3
    N, K = dy.shape[1], x.shape[1]
    pts = stratified_points(N, K, 2000, seed=13)
    err, y, exact = _wgrad_case(dy, x, pts=pts, pow2=pow2)
    assert normwise(y, exact) <= TOL_F32


# ------------------------------------------------------------------------------------------------
# Grouped (MoE experts)
# ------------------------------------------------------------------------------------------------

def _grouped_case(x, w, offsets, bf16=True, pts=None, pow2=False):
    xq, sx = fg.fg_quantize_act_1x128(to_dev(x), pow2=pow2)
    G, N, K = w.shape
    wq = torch.empty((G, N, K), dtype=torch.uint8, device=device())
    sw = torch.empty((G, (N + 127) // 128, K // 128), dtype=torch.float32, device=device())
    wd = to_dev(w)
    for g in range(G):
        fg.fg_quantize_w_128x128(wd[g], q=wq[g], scales=sw[g], pow2=pow2)
    off = torch.from_numpy(np.asarray(offsets, np.int32)).to(device())
    y = nan_like_out((x.shape[0], N), torch.bfloat16 if bf16 else torch.float32)
    fg.fg_fp8_grouped_gemm(xq, sx, wq, sw, off, y=y, pow2=pow2)
    torch.cuda.synchronize()
    assert_all_written(y, "grouped")
    xq_o, sx_o = oracle.quantize_act_1x128(bits(x), 0, pow2)
    assert np.array_equal(np_u8(xq), xq_o)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), sx_o.view(np.uint32)), "activation scales"
    wo = [oracle.quantize_w_128x128(bits(w[g]), pow2) for g in range(G)]
    wq_o, sw_o = np.stack([a for a, _ in wo]), np.stack([b for _, b in wo])
    assert np.array_equal(np_u8(wq), wq_o)
    assert np.array_equal(sw.cpu().numpy().view(np.uint32), sw_o.view(np.uint32)), "weight scales"
    prom, exact = oracle.gemm_grouped(xq_o, sx_o, wq_o, sw_o, offsets, out_bf16=bf16, pts=pts)
    yo = _out_np(y, bf16).reshape(-1)
    yo = yo if pts is None else yo[pts]
    return _cmp(yo, prom, bf16), yo, exact


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("tile", TILES, indirect=True)
def test_grouped_small_with_empty_groups(bf16, pow2, tile):
    device()
    rng = np.random.default_rng(21)
    offsets = [0, 0, 300, 301, 301, 700, 957]            # empty groups at 0 and 3, a 1-row group
    T, K, N = offsets[-1], 256, 136
    x = _rand_act(rng, T, K)
    w = wl.normal_bf16(rng, (len(offsets) - 1, N, K), 0.02)
    _grouped_case(x, w, offsets, bf16, pow2=pow2)


def test_grouped_moe_share_full_size_sampled(moe_share):
    device()
    d = moe_share
    T = int(d["offsets"][-1])
    assert T == wl.MOE_TOKENS * wl.MOE_TOPK
    pts = stratified_points(T, wl.MOE_INTER, 2000, seed=14)
    err, y, exact = _grouped_case(d["x"], d["w_up"], d["offsets"], bf16=True, pts=pts)
    assert normwise(bf16_bits_to_f64(y), exact) <= TOL_BF16


def test_grouped_moe_down_projection_full_size_sampled(moe_share):
    """The down-projection at all 65536 routed rows: H [65536, 2048] . W_down[e]^T -> [65536, 7168]."""
    device()
    d = moe_share
    T = int(d["offsets"][-1])
    assert T == wl.MOE_TOKENS * wl.MOE_TOPK
    pts = stratified_points(T, wl.MOE_HIDDEN, 2000, seed=15)
    err, y, exact = _grouped_case(d["h"], d["w_down"], d["offsets"], bf16=True, pts=pts)
    assert normwise(bf16_bits_to_f64(y), exact) <= TOL_BF16


# ------------------------------------------------------------------------------------------------
# MoE backward: grouped Dgrad and grouped Wgrad, checked per expert against the oracle's Dgrad/Wgrad of
# that expert's slice
# ------------------------------------------------------------------------------------------------

def _grouped_dgrad_case(dy, w, offsets, bf16=False, pts_per_group=None, pow2=False):
    dyq, sdy = fg.fg_quantize_act_1x128(to_dev(dy), pow2=pow2)
    G, N, K = w.shape
    wq = torch.empty((G, N, K), dtype=torch.uint8, device=device())
    sw = torch.empty((G, N // 128, (K + 127) // 128), dtype=torch.float32, device=device())
    wd = to_dev(w)
    for g in range(G):
        fg.fg_quantize_w_128x128(wd[g], q=wq[g], scales=sw[g], pow2=pow2)
    off = torch.from_numpy(np.asarray(offsets, np.int32)).to(device())
    dx = nan_like_out((dy.shape[0], K), torch.bfloat16 if bf16 else torch.float32)
    fg.fg_fp8_grouped_gemm_dgrad(dyq, sdy, wq, sw, off, dx=dx, pow2=pow2)
    torch.cuda.synchronize()
    assert_all_written(dx, "grouped dgrad")
    dyq_o, sdy_o = oracle.quantize_act_1x128(bits(dy), 0, pow2)
    assert np.array_equal(np_u8(dyq), dyq_o)
    out = _out_np(dx, bf16)
    errs = []
    for g in range(G):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 == r0:
            continue
        wq_o, sw_o = oracle.quantize_w_128x128(bits(w[g]), pow2)
        pts = None if pts_per_group is None else stratified_points(r1 - r0, K, pts_per_group, seed=31 + g)
        prom, _ = oracle.gemm_dgrad(dyq_o[r0:r1], np.ascontiguousarray(sdy_o[:, r0:r1]), wq_o, sw_o, out_bf16=bf16,
                                    pts=pts)
        yo = out[r0:r1].reshape(-1)
        yo = yo if pts is None else yo[pts]
        errs.append(_cmp(yo, prom, bf16))
    return errs


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("tile", TILES, indirect=True)
def test_grouped_dgrad_small_with_empty_groups(bf16, pow2, tile):
    device()
    rng = np.random.default_rng(22)
    offsets = [0, 0, 300, 301, 301, 700, 957]
    T, N, K = offsets[-1], 256, 384
    dy = _rand_act(rng, T, N, 1e-3)
    w = wl.normal_bf16(rng, (len(offsets) - 1, N, K), 0.02)
    _grouped_dgrad_case(dy, w, offsets, bf16, pow2=pow2)


@pytest.mark.parametrize("pow2", [False, True])
def test_grouped_dgrad_moe_share_sampled(pow2):
    device()
    d = wl.moe_backward_inputs()
    _grouped_dgrad_case(d["dy"], d["w_up"], d["offsets"], pts_per_group=300, pow2=pow2)


def _grouped_wgrad_case(dy, x, offsets, init=None, pts_per_group=None, pow2=False):
    dytq, sdyt = fg.fg_quantize_act_1x128(to_dev(dy), axis=fg.FG_ALONG_ROWS, pow2=pow2)
    xtq, sxt = fg.fg_quantize_act_1x128(to_dev(x), axis=fg.FG_ALONG_ROWS, pow2=pow2)
    T, N = dy.shape
    K = x.shape[1]
    G = len(offsets) - 1
    off = torch.from_numpy(np.asarray(offsets, np.int32)).to(device())
    if init is not None:
        dw = fg.fg_fp8_grouped_gemm_wgrad(dytq, sdyt, xtq, sxt, off, dw=to_dev(torch.from_numpy(init)), accumulate=True,
                                          pow2=pow2)
    else:
        dw = nan_like_out((G, N, K), torch.float32)
        fg.fg_fp8_grouped_gemm_wgrad(dytq, sdyt, xtq, sxt, off, dw=dw, pow2=pow2)
    torch.cuda.synchronize()
    assert_all_written(dw, "grouped wgrad")
    dytq_o, sdyt_o = oracle.quantize_act_1x128(bits(dy), 1, pow2)
    xtq_o, sxt_o = oracle.quantize_act_1x128(bits(x), 1, pow2)
    assert np.array_equal(np_u8(dytq), dytq_o) and np.array_equal(np_u8(xtq), xtq_o)
    out = dw.cpu().numpy()
    errs = []
    for g in range(G):
        t0, t1 = int(offsets[g]), int(offsets[g + 1])
        pts = None if pts_per_group is None else stratified_points(N, K, pts_per_group, seed=41 + g)
        init_g = None if init is None else (init[g].reshape(-1) if pts is None else init[g].reshape(-1)[pts])
        prom, _ = oracle.gemm_wgrad(np.ascontiguousarray(dytq_o[:, t0:t1]), np.ascontiguousarray(sdyt_o[t0 // 128: t1 // 128]),
                                    np.ascontiguousarray(xtq_o[:, t0:t1]), np.ascontiguousarray(sxt_o[t0 // 128: t1 // 128]),
                                    dw_init=init_g, pts=pts)
        yo = out[g].reshape(-1)
        yo = yo if pts is None else yo[pts]
        if t1 == t0 and init is None:
            assert not np.any(yo), "empty group must write zeros"
            continue
        errs.append(_cmp(yo, prom, False))
    return errs


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("tile", TILES, indirect=True)
def test_grouped_wgrad_small_with_empty_group(pow2, tile):
    device()
    rng = np.random.default_rng(23)
    offsets = [0, 128, 128, 512, 640]                    # an empty group
    T, N, K = offsets[-1], 200, 136
    _grouped_wgrad_case(_rand_act(rng, T, N, 1e-3), _rand_act(rng, T, K), offsets, pow2=pow2)


@pytest.mark.parametrize("pow2", [False, True])
def test_grouped_wgrad_accumulate(pow2):
    device()
    rng = np.random.default_rng(24)
    offsets = [0, 256, 256, 384]
    T, N, K = offsets[-1], 256, 264
    init = (rng.standard_normal((3, N, K)) * 1e-3).astype(np.float32)
    _grouped_wgrad_case(_rand_act(rng, T, N, 1e-3), _rand_act(rng, T, K), offsets, init=init, pow2=pow2)


@pytest.mark.parametrize("pow2", [False, True])
def test_grouped_wgrad_moe_share_sampled(pow2):
    device()
    d = wl.moe_backward_inputs()
    _grouped_wgrad_case(d["dy"], d["x"], d["offsets"], pts_per_group=300, pow2=pow2)


# ------------------------------------------------------------------------------------------------
# The two workgroup shapes give bit-identical results
# ------------------------------------------------------------------------------------------------

def test_grouped_offsets_clamped_on_device():
    """Device offsets outside [0, T] are clamped into it: offsets that start below 0 and end past T give the
    same outputs, bit for bit, as the offsets they clamp to, and nothing outside the operands is touched."""
    device()
    rng = np.random.default_rng(82)
    T, N, K = 300, 136, 256
    x = to_dev(_rand_act(rng, T, K))
    w = to_dev(wl.normal_bf16(rng, (2, N, K), 0.02))
    xq, sx = fg.fg_quantize_act_1x128(x)
    wq = torch.stack([fg.fg_quantize_w_128x128(w[g])[0] for g in range(2)])
    sw = torch.stack([fg.fg_quantize_w_128x128(w[g])[1] for g in range(2)])
    good = torch.tensor([0, 100, T], dtype=torch.int32, device=device())
    bad = torch.tensor([-50, 100, T + 1000], dtype=torch.int32, device=device())
    y_good = fg.fg_fp8_grouped_gemm(xq, sx, wq, sw, good, out_dtype=torch.float32)
    y_bad = fg.fg_fp8_grouped_gemm(xq, sx, wq, sw, bad, out_dtype=torch.float32)
    # grouped Dgrad: dY [T, 256] against W [2][256][K]
    dy = to_dev(_rand_act(rng, T, 256, 1e-3))
    wd = to_dev(wl.normal_bf16(rng, (2, 256, K), 0.02))
    dyq, sdy = fg.fg_quantize_act_1x128(dy)
    wdq = torch.stack([fg.fg_quantize_w_128x128(wd[g])[0] for g in range(2)])
    swd = torch.stack([fg.fg_quantize_w_128x128(wd[g])[1] for g in range(2)])
    dx_good = fg.fg_fp8_grouped_gemm_dgrad(dyq, sdy, wdq, swd, good)
    dx_bad = fg.fg_fp8_grouped_gemm_dgrad(dyq, sdy, wdq, swd, bad)
    # grouped Wgrad: token segments in multiples of 128
    Tw = 384
    dyw = to_dev(_rand_act(rng, Tw, 200, 1e-3))
    xw = to_dev(_rand_act(rng, Tw, 136))
    dytq, sdyt = fg.fg_quantize_act_1x128(dyw, axis=fg.FG_ALONG_ROWS)
    xtq, sxt = fg.fg_quantize_act_1x128(xw, axis=fg.FG_ALONG_ROWS)
    goodw = torch.tensor([0, 128, Tw], dtype=torch.int32, device=device())
    badw = torch.tensor([-128, 128, Tw + 256], dtype=torch.int32, device=device())
    dw_good = fg.fg_fp8_grouped_gemm_wgrad(dytq, sdyt, xtq, sxt, goodw)
    dw_bad = fg.fg_fp8_grouped_gemm_wgrad(dytq, sdyt, xtq, sxt, badw)
    torch.cuda.synchronize()
    for name, a, b in (("fprop", y_good, y_bad), ("dgrad", dx_good, dx_bad), ("wgrad", dw_good, dw_bad)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), name


# ------------------------------------------------------------------------------------------------
# Power-of-2 mode handed scales that are not powers of two: NaN outputs, not silently wrong sums
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("tile", FPROP_TILES, indirect=True)
def test_pow2_mode_poisons_tiles_with_other_scales(tile):
    """Power-of-2 codes and scales, with one activation row's scale given mantissa bits: every output of
    the wave tiles that read that scale is NaN, every other output equals the clean run bit for bit."""
    device()
    rng = np.random.default_rng(91)
    M, N, K = 300, 520, 384
    xq, sx = fg.fg_quantize_act_1x128(to_dev(_rand_act(rng, M, K)), pow2=True)
    wq, sw = fg.fg_quantize_w_128x128(to_dev(wl.normal_bf16(rng, (N, K), 0.02)), pow2=True)
    clean = fg.fg_fp8_gemm_fprop(xq, sx, wq, sw, out_dtype=torch.float32, pow2=True)
    bad_sx = sx.clone()
    bad_sx[1, 5] *= 1.5                                  # row 5, second 128-block: not a power of two
    y = fg.fg_fp8_gemm_fprop(xq, bad_sx, wq, sw, out_dtype=torch.float32, pow2=True)
    torch.cuda.synchronize()
    assert torch.isnan(y[5]).all(), "the row whose scale has mantissa bits must be NaN"
    assert torch.isfinite(y[128:]).all() and torch.equal(y[128:].view(torch.int32), clean[128:].view(torch.int32))
    finite_rows = torch.isfinite(y).all(dim=1)
    assert torch.equal(y[finite_rows].view(torch.int32), clean[finite_rows].view(torch.int32))


def test_pow2_mode_with_fp32_scales_is_nan_everywhere():
    """FP32-mode scales (almost none a power of two) declared as power-of-2 scales: every GEMM entry point
    returns NaN outputs (and NaN codes and scales from the quantizing Fprop)."""
    device()
    rng = np.random.default_rng(92)
    M, N, K = 256, 384, 512
    x, w = to_dev(_rand_act(rng, M, K)), to_dev(wl.normal_bf16(rng, (N, K), 0.02))
    dy = to_dev(_rand_act(rng, M, N, 1e-3))
    xq, sx = fg.fg_quantize_act_1x128(x)
    wq, sw = fg.fg_quantize_w_128x128(w)
    dyq, sdy = fg.fg_quantize_act_1x128(dy)
    dytq, sdyt = fg.fg_quantize_act_1x128(dy, axis=fg.FG_ALONG_ROWS)
    xtq, sxt = fg.fg_quantize_act_1x128(x, axis=fg.FG_ALONG_ROWS)
    off = torch.tensor([0, 100, M], dtype=torch.int32, device=device())
    offw = torch.tensor([0, 128, M], dtype=torch.int32, device=device())
    outs = {
        "fprop": fg.fg_fp8_gemm_fprop(xq, sx, wq, sw, out_dtype=torch.float32, pow2=True),
        "fprop_bf16": fg.fg_fp8_gemm_fprop(xq, sx, wq, sw, pow2=True),
        "dgrad": fg.fg_fp8_gemm_dgrad(dyq, sdy, wq, sw, pow2=True),
        "wgrad": fg.fg_fp8_gemm_wgrad(dytq, sdyt, xtq, sxt, pow2=True),
        "grouped": fg.fg_fp8_grouped_gemm(xq, sx, torch.stack([wq, wq]), torch.stack([sw, sw]), off, pow2=True),
        "grouped_dgrad": fg.fg_fp8_grouped_gemm_dgrad(dyq, sdy, torch.stack([wq, wq]), torch.stack([sw, sw]), off,
                                                      pow2=True),
        "grouped_wgrad": fg.fg_fp8_grouped_gemm_wgrad(dytq, sdyt, xtq, sxt, offw, pow2=True),
    }
    yq, sy = fg.fg_fp8_gemm_fprop_quant(xq, sx, wq, sw, pow2=True)
    torch.cuda.synchronize()
    for name, t in outs.items():
        assert torch.isnan(t.float()).all(), name
    assert torch.isnan(sy).all()
    assert bool(((yq & 0x7F) == 0x7F).all()), "quantizing Fprop: NaN codes"


@pytest.mark.parametrize("M,N,K", [(300, 520, 640), (300, 576, 384), (513, 1152, 256)])
@pytest.mark.parametrize("pow2", [False, True])
def test_fprop_wide_tile_bit_identical(M, N, K, pow2, monkeypatch):
    """Fprop on 256x288 tiles (each wave keeps its A fragments and streams B) gives the 256x256 shape's
    outputs bit for bit, for both output types: ragged rows, and columns that end inside a wave tile, on a
    wave-tile boundary, or on a workgroup-tile boundary (staged and direct stores)."""
    device()
    rng = np.random.default_rng(M + N + K)
    xq, sx = fg.fg_quantize_act_1x128(to_dev(_rand_act(rng, M, K)), pow2=pow2)
    wq, sw = fg.fg_quantize_w_128x128(to_dev(wl.normal_bf16(rng, (N, K), 0.02)), pow2=pow2)
    outs = {}
    for val in ("256x256", "256x288"):
        monkeypatch.setenv("FG_GEMM_TILE", val)
        outs[val] = [fg.fg_fp8_gemm_fprop(xq, sx, wq, sw, y=nan_like_out((M, N), dt), pow2=pow2)
                     for dt in (torch.float32, torch.bfloat16)]
        torch.cuda.synchronize()
    for a, b in zip(outs["256x256"], outs["256x288"]):
        assert_all_written(b, "fprop 256x288")
        iv = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(a.view(iv), b.view(iv)), a.dtype


@pytest.mark.parametrize("pow2", [False, True])
def test_tile_shapes_bit_identical(pow2, monkeypatch):
    """Every output element goes through the same instructions in the same order under either workgroup
    shape, so Fprop (both output types), Dgrad, Wgrad (plain and accumulating) and grouped Fprop outputs
    must match bit for bit (ragged shapes)."""
    device()
    rng = np.random.default_rng(81)
    M, N, K = 300, 520, 640
    x = to_dev(_rand_act(rng, M, K))
    w = to_dev(wl.normal_bf16(rng, (N, K), 0.02))
    dy = to_dev(wl.normal_bf16(rng, (M, 384), 1e-3))
    wd = to_dev(wl.normal_bf16(rng, (384, K), 0.02))
    xq, sx = fg.fg_quantize_act_1x128(x, pow2=pow2)
    wq, sw = fg.fg_quantize_w_128x128(w, pow2=pow2)
    dyq, sdy = fg.fg_quantize_act_1x128(dy, pow2=pow2)
    wdq, swd = fg.fg_quantize_w_128x128(wd, pow2=pow2)
    xr = to_dev(_rand_act(rng, 384, 264))
    dyr = to_dev(wl.normal_bf16(rng, (384, 200), 1e-3))
    dytq, sdyt = fg.fg_quantize_act_1x128(dyr, axis=fg.FG_ALONG_ROWS, pow2=pow2)
    xtq, sxt = fg.fg_quantize_act_1x128(xr, axis=fg.FG_ALONG_ROWS, pow2=pow2)
    off = torch.tensor([0, 100, 100, 300], dtype=torch.int32, device=device())
    wg, swg = torch.stack([wq, wq, wq]), torch.stack([sw, sw, sw])
    dw0 = torch.randn((200, 264), dtype=torch.float32, device=device())
    outs = {}
    for val in ("256x192", "256x256"):
        monkeypatch.setenv("FG_GEMM_TILE", val)
        dw_acc = dw0.clone()
        outs[val] = [fg.fg_fp8_gemm_fprop(xq, sx, wq, sw, out_dtype=torch.float32, pow2=pow2),
                     fg.fg_fp8_gemm_fprop(xq, sx, wq, sw, out_dtype=torch.bfloat16, pow2=pow2),
                     fg.fg_fp8_gemm_dgrad(dyq, sdy, wdq, swd, pow2=pow2),
                     fg.fg_fp8_gemm_wgrad(dytq, sdyt, xtq, sxt, pow2=pow2),
                     fg.fg_fp8_gemm_wgrad(dytq, sdyt, xtq, sxt, dw=dw_acc, accumulate=True, pow2=pow2),
                     fg.fg_fp8_grouped_gemm(xq, sx, wg, swg, off, out_dtype=torch.float32, pow2=pow2)]
        torch.cuda.synchronize()
    names = ("fprop", "fprop_bf16", "dgrad", "wgrad", "wgrad_accumulate", "grouped")
    for name, a, b in zip(names, outs["256x192"], outs["256x256"]):
        assert torch.equal(a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32),
                           b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32)), name
