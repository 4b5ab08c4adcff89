"""GPU parity of per-tensor scaling (the contrast baseline) and its accuracy against the 1x128 / 128x128
tiles.

fg_amax_bf16 and fg_quantize_per_tensor are compared bit for bit with the oracle (max-abs, codes and the
broadcast scales) for current scaling (history = the tensor's own max-abs), delayed scaling with
histories below (saturation) and above the current max-abs, empty and non-bf16 histories, scales below
2^-100, inputs whose quotient overflows fp32, both scale layouts, ragged and full-size shapes. The
accuracy legs run the same block-scaled Fprop on per-tensor and on fine-grained codes and report the
error of each against the exact product of the unquantized bf16 operands.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_amax_amd as fg
import oracle
from fp8_fine_grained_amax_amd import workloads as wl
from tests.gpu_util import TOL_F32, bits, device, normwise, np_u8, sample_points, to_dev

pytestmark = pytest.mark.gpu


def _hist(vals):
    return torch.tensor(np.asarray(vals, np.float32).reshape(-1), dtype=torch.float32, device=device())


def _check_quant(xb_t, hist_vals, pow2, layout, amax_out=None):
    hist = _hist(hist_vals)
    q, s = fg.fg_quantize_per_tensor(xb_t, hist, pow2=pow2, layout=layout, amax_out=amax_out)
    torch.cuda.synchronize()
    q_o, s_o = oracle.quantize_per_tensor(bits(xb_t), np.asarray(hist_vals, np.float32), pow2, layout)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_o.view(np.uint32)), "scales differ from the oracle's"
    bad = np.argwhere(np_u8(q) != q_o)
    assert bad.size == 0, f"{len(bad)} codes differ from the oracle's, first at {bad[:4].tolist()}"
    return np_u8(q), s.cpu().numpy()


@pytest.mark.parametrize("rows,cols,ld", [(1, 8, 8), (5, 136, 136), (300, 1024, 1032), (4096, 7168, 7168)])
def test_amax_exact(rows, cols, ld):
    device()
    rng = np.random.default_rng(rows + cols)
    full = wl.normal_bf16(rng, (rows, ld), 1.0, outlier_channels=min(3, ld // 8), outlier_scale=50.0)
    x = to_dev(full)[:, :cols]
    a = fg.fg_amax_bf16(x)
    torch.cuda.synchronize()
    ref = oracle.amax_bf16(np.ascontiguousarray(bits(full)[:, :cols]))
    assert a.item() == ref
    # folds into the value already there
    b = torch.full((1,), 2.0 * ref, dtype=torch.float32, device=device())
    fg.fg_amax_bf16(x, amax=b)
    torch.cuda.synchronize()
    assert b.item() == np.float32(2.0 * ref)


@pytest.mark.parametrize("layout", [fg.FG_LAYOUT_ACT_1x128, fg.FG_LAYOUT_W_128x128])
@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("rows,cols", [(1, 128), (130, 256), (300, 1024), (4096, 7168)])
def test_current_scaling_exact(rows, cols, pow2, layout):
    device()
    rng = np.random.default_rng(rows * 3 + cols + pow2)
    x = to_dev(wl.normal_bf16(rng, (rows, cols), 1.0, outlier_channels=min(8, cols // 128), outlier_scale=20.0))
    amax = fg.fg_amax_bf16(x)
    torch.cuda.synchronize()
    q, _ = _check_quant(x, [amax.item()], pow2, layout)
    if not pow2:
        assert (q & 0x7F).max() == 0x7E


@pytest.mark.parametrize("pow2", [False, True])
def test_delayed_scaling_exact_and_records_amax(pow2):
    device()
    rng = np.random.default_rng(91)
    x = to_dev(wl.normal_bf16(rng, (520, 768), 1.0, outlier_channels=4, outlier_scale=20.0))
    a = oracle.amax_bf16(bits(x))
    for hist in ([0.3 * a, 0.5 * a, -0.45 * a],            # below the current max-abs: the top saturates
                 [a * 3.0, a],                             # above: nothing saturates
                 [1.0 + 2.0 ** -10, 0.7],                  # between bf16 numbers: rounded up
                 []):                                      # empty: scale 1
        out = torch.zeros((1,), dtype=torch.float32, device=device())
        q, _ = _check_quant(x, hist, pow2, fg.FG_LAYOUT_ACT_1x128, amax_out=out)
        assert out.item() == a
    # saturation did happen in the first case
    q, s = _check_quant(x, [0.5 * a], pow2, fg.FG_LAYOUT_ACT_1x128)
    assert ((q & 0x7F) == 0x7E).sum() > 1


def test_tiny_scales_and_overflowing_quotients():
    device()
    rng = np.random.default_rng(92)
    # whole tensor tiny: a scale below 2^-100 (the 2^64-shifted quotient form)
    xt = to_dev(wl.to_bf16(rng.standard_normal((64, 256), dtype=np.float32) * np.float32(1e-30)))
    amax = fg.fg_amax_bf16(xt)
    torch.cuda.synchronize()
    _, s = _check_quant(xt, [amax.item()], False, fg.FG_LAYOUT_ACT_1x128)
    assert s[0, 0] < 2.0 ** -100
    # histories far below the data: x * (1/s) overflows fp32 in both quotient forms; all saturate
    xb = to_dev(wl.to_bf16(rng.standard_normal((64, 256), dtype=np.float32) * np.float32(1e20)))
    for hist in ([1e-20], [1e-35]):
        q, _ = _check_quant(xb, hist, False, fg.FG_LAYOUT_ACT_1x128)
        assert ((q & 0x7F) == 0x7E).mean() > 0.99
    q, _ = _check_quant(xb, [1e-35], True, fg.FG_LAYOUT_ACT_1x128)


def _exact_fprop(x, w):
    xf = oracle.bf16_bits_to_f32(bits(x)).astype(np.float64)
    wf = oracle.bf16_bits_to_f32(bits(w)).astype(np.float64)
    return xf @ wf.T


def _fprop_errors(x, w, exact):
    """Normwise error against the exact product, for fine-grained and per-tensor (current) codes."""
    xq, sx = fg.fg_quantize_act_1x128(x)
    wq, sw = fg.fg_quantize_w_128x128(w)
    y_fg = fg.fg_fp8_gemm_fprop(xq, sx, wq, sw, out_dtype=torch.float32)
    ax, aw = fg.fg_amax_bf16(x), fg.fg_amax_bf16(w)
    xp, sxp = fg.fg_quantize_per_tensor(x, ax)
    wp, swp = fg.fg_quantize_per_tensor(w, aw, layout=fg.FG_LAYOUT_W_128x128)
    y_pt = fg.fg_fp8_gemm_fprop(xp, sxp, wp, swp, out_dtype=torch.float32)
    torch.cuda.synchronize()
    # the per-tensor path's codes are the oracle's, and the GEMM on them is within the GEMM tolerance
    xp_o, sxp_o = oracle.quantize_per_tensor(bits(x), [ax.item()], False, 0)
    wp_o, swp_o = oracle.quantize_per_tensor(bits(w), [aw.item()], False, 1)
    assert np.array_equal(np_u8(xp), xp_o) and np.array_equal(np_u8(wp), wp_o)
    pts = sample_points(x.shape[0], w.shape[0], 3000, seed=95)
    prom, _ = oracle.gemm_fprop(xp_o, sxp_o, wp_o, swp_o, pts=pts, want_exact=False)
    assert normwise(y_pt.cpu().numpy().reshape(-1)[pts], prom) <= TOL_F32
    return normwise(y_fg.cpu().numpy(), exact), normwise(y_pt.cpu().numpy(), exact)


def test_accuracy_fine_grained_vs_per_tensor():
    """X [1024, 7168] and W [2048, 7168] with the dense-MLP distributions (1% of channels x20), and the same
    with 0.1% of channels x10^4: normwise error of Fprop against the exact product of the bf16 operands."""
    device()
    rng = np.random.default_rng(93)
    w = to_dev(wl.normal_bf16(rng, (2048, 7168), 0.006))
    rows = {}
    for name, n_out, scale in (("outliers x20 on 1% of channels", 72, 20.0),
                               ("outliers x10^4 on 0.1% of channels", 7, 1e4)):
        x = to_dev(wl.normal_bf16(rng, (1024, 7168), 1.0, outlier_channels=n_out, outlier_scale=scale))
        exact = _exact_fprop(x, w)
        rows[name] = _fprop_errors(x, w, exact)
        print(f"\n[per-tensor] {name}: fine-grained {rows[name][0]:.3e}, per-tensor {rows[name][1]:.3e}")
    for e_fg, e_pt in rows.values():
        assert e_fg < 0.05 and e_pt > 1.2 * e_fg


def test_accuracy_delayed_scaling_spike():
    """Delayed scaling over a short run of steps: the history holds the previous steps' max-abs values, and
    a step whose max-abs jumps 8x above them saturates its outliers; the current-scaling and fine-grained
    errors of the same step are reported beside it."""
    device()
    rng = np.random.default_rng(94)
    w = to_dev(wl.normal_bf16(rng, (1024, 2048), 0.02))
    wq, sw = fg.fg_quantize_w_128x128(w)
    H = 4
    hist = torch.zeros((H,), dtype=torch.float32, device=device())
    errs = []
    for step in range(6):
        spike = 8.0 if step == 5 else 1.0
        x = to_dev(wl.normal_bf16(rng, (512, 2048), 1.0, outlier_channels=16, outlier_scale=20.0 * spike))
        cur = torch.zeros((1,), dtype=torch.float32, device=device())
        xq, sx = fg.fg_quantize_per_tensor(x, hist if step > 0 else fg.fg_amax_bf16(x), amax_out=cur)
        q_o, _ = oracle.quantize_per_tensor(bits(x), hist.cpu().numpy() if step > 0 else [cur.item()], False, 0)
        torch.cuda.synchronize()
        assert np.array_equal(np_u8(xq), q_o)
        hist[step % H] = cur[0]
        y = fg.fg_fp8_gemm_fprop(xq, sx, wq, sw, out_dtype=torch.float32)
        torch.cuda.synchronize()
        exact = _exact_fprop(x, w)
        errs.append(normwise(y.cpu().numpy(), exact))
    xq_c, sx_c = fg.fg_quantize_per_tensor(x, fg.fg_amax_bf16(x))
    xq_f, sx_f = fg.fg_quantize_act_1x128(x)
    e_cur = normwise(fg.fg_fp8_gemm_fprop(xq_c, sx_c, wq, sw, out_dtype=torch.float32).cpu().numpy(), exact)
    e_fg = normwise(fg.fg_fp8_gemm_fprop(xq_f, sx_f, wq, sw, out_dtype=torch.float32).cpu().numpy(), exact)
    print(f"\n[delayed] per-step errors {', '.join(f'{e:.3e}' for e in errs)}; spike step: "
          f"current per-tensor {e_cur:.3e}, fine-grained {e_fg:.3e}")
    assert errs[5] > 4 * max(errs[1:5]) and errs[5] > 4 * e_cur
