"""GPU parity: the HIP quantizers against the CPU oracle, bit-exact on codes and scales.

Workloads are the seeded synthetic inputs (full sizes of the DeepSeek-V3-like Linear and its backward
pair, the MoE share, the tiny case) plus edge cases: ragged rows/columns, padded row strides, zero and
subnormal tiles, signed zeros, bf16 extremes, tiny scales, and a sweep over every finite bf16 value.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_amax_amd as fg
import oracle
from fp8_fine_grained_amax_amd import workloads as wl
from tests.gpu_util import bits, device, np_u8, to_dev

pytestmark = pytest.mark.gpu


def _check_act(x_cpu, axis, pow2, ld_pad=0):
    xb = bits(x_cpu)
    x = to_dev(x_cpu)
    if ld_pad:
        big = torch.zeros((x.shape[0], x.shape[1] + ld_pad), dtype=torch.bfloat16, device=x.device)
        big[:, : x.shape[1]] = x
        x = big[:, : x_cpu.shape[1]]
    q, s = fg.fg_quantize_act_1x128(x, axis=axis, pow2=pow2)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_act_1x128(xb, axis, pow2)
    q_gpu, s_gpu = np_u8(q), s.cpu().numpy()
    assert np.array_equal(s_gpu.view(np.uint32), s_ref.view(np.uint32)), "scales differ"
    bad = np.argwhere(q_gpu != q_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:5].tolist()}"


def _check_w(w_cpu, pow2):
    q, s = fg.fg_quantize_w_128x128(to_dev(w_cpu), pow2=pow2)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_w_128x128(bits(w_cpu), pow2)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), "scales differ"
    assert np.array_equal(np_u8(q), q_ref), "codes differ"


@pytest.mark.parametrize("pow2", [False, True])
def test_tiny_config(pow2):
    device()
    x, w = wl.tiny_fprop()
    _check_act(x, fg.FG_ALONG_COLS, pow2)
    _check_w(w, pow2)


@pytest.fixture(scope="module")
def dsv3():
    device()
    x, w = wl.dsv3_fprop()
    dy = wl.dsv3_backward_dy()
    return x, w, dy


@pytest.mark.parametrize("pow2", [False, True])
def test_dsv3_activation_rowwise(dsv3, pow2):
    _check_act(dsv3[0], fg.FG_ALONG_COLS, pow2)


def test_dsv3_weight_blocks(dsv3):
    _check_w(dsv3[1], False)


def test_dsv3_weight_blocks_pow2(dsv3):
    _check_w(dsv3[1], True)


def test_dsv3_backward_dy_rowwise(dsv3):
    _check_act(dsv3[2], fg.FG_ALONG_COLS, False)


def test_dsv3_backward_token_dim(dsv3):
    _check_act(dsv3[2], fg.FG_ALONG_ROWS, False)      # dY^T for Wgrad
    _check_act(dsv3[0], fg.FG_ALONG_ROWS, False)      # X^T for Wgrad


@pytest.mark.parametrize("pow2", [False, True])
def test_moe_share_inputs_full_size(moe_share, pow2):
    """One GPU's MoE share at its stated size: X [65536, 7168] and H [65536, 2048] (the up- and
    down-projection inputs), codes and scales bit-exact, and every expert's W_up and W_down blocks."""
    device()
    d = moe_share
    assert d["x"].shape == (wl.MOE_TOKENS * wl.MOE_TOPK, wl.MOE_HIDDEN)
    assert d["h"].shape == (wl.MOE_TOKENS * wl.MOE_TOPK, wl.MOE_INTER)
    _check_act(d["x"], fg.FG_ALONG_COLS, pow2)
    _check_act(d["h"], fg.FG_ALONG_COLS, pow2)
    for e in range(wl.MOE_EXPERTS):
        _check_w(d["w_up"][e], pow2)
        _check_w(d["w_down"][e], pow2)


@pytest.mark.parametrize("rows,cols,ld_pad", [(1, 128, 0), (37, 384, 8), (65, 1024, 0), (1000, 256, 24)])
@pytest.mark.parametrize("pow2", [False, True])
def test_rowwise_ragged_and_strided(rows, cols, ld_pad, pow2):
    device()
    rng = np.random.default_rng(rows * 7 + cols)
    x = wl.normal_bf16(rng, (rows, cols), 3.0, outlier_channels=2, outlier_scale=100.0)
    _check_act(x, fg.FG_ALONG_COLS, pow2, ld_pad)


@pytest.mark.parametrize("rows,cols,ld_pad", [(128, 8, 0), (256, 200, 8), (384, 72, 0), (128, 1032, 16)])
@pytest.mark.parametrize("pow2", [False, True])
def test_token_dim_ragged_and_strided(rows, cols, ld_pad, pow2):
    device()
    rng = np.random.default_rng(rows + cols * 3)
    x = wl.normal_bf16(rng, (rows, cols), 0.5, outlier_channels=1, outlier_scale=50.0)
    _check_act(x, fg.FG_ALONG_ROWS, pow2, ld_pad)


@pytest.mark.parametrize("n,k", [(1, 128), (300, 256), (129, 640)])
@pytest.mark.parametrize("pow2", [False, True])
def test_weight_ragged(n, k, pow2):
    device()
    rng = np.random.default_rng(n + k)
    _check_w(wl.normal_bf16(rng, (n, k), 0.02), pow2)


def _special_tiles():
    """Rows of 128 bf16 values exercising the scale and rounding edge cases."""
    rows = []
    z = np.zeros(128, np.uint16)
    rows.append(z.copy())                                           # all +0: scale 1
    r = z.copy(); r[::2] = 0x8000; rows.append(r)                   # mix of -0 and +0
    r = z.copy(); r[5] = 0x0001; r[9] = 0x8003; rows.append(r)      # bf16 subnormals only (tiny scale)
    r = z.copy(); r[0] = 0x7F7F; r[1] = 0xFF7F; r[2] = 0x0001; rows.append(r)   # bf16 max and min
    r = z.copy(); r[0] = 0x0080; r[1] = 0x8080; r[2] = 0x0001; rows.append(r)   # FLT_MIN-sized amax
    r = z.copy(); r[0] = 0x43E0; r[1:8] = [0x3A80, 0x3AC0, 0x3B40, 0x3B00, 0xBA80, 0x8000, 0x3F80]; rows.append(r)  # 448 & ties
    r = z.copy(); r[:] = 0x3F80; rows.append(r)                      # constant tile
    r = z.copy(); r[0] = 0x11E0; r[1] = 0x1100; r[2] = 0x9180; rows.append(r)   # amax = 448 * 2^-100: s = 2^-100
    r = z.copy(); r[0] = 0x11DF; r[1] = 0x0080; r[2] = 0x8C00; r[3] = 0x0001; rows.append(r)  # s just below 2^-100
    r = z.copy(); r[0] = 0x0D00; r[1] = 0x0080; r[2] = 0x8C00; rows.append(r)   # s < 2^-100 (pre-scaled path)
    return np.stack(rows)


@pytest.mark.parametrize("pow2", [False, True])
def test_special_value_tiles(pow2):
    device()
    t = _special_tiles()
    x = torch.from_numpy(t.view(np.int16)).view(torch.bfloat16)
    _check_act(x, fg.FG_ALONG_COLS, pow2)


def test_special_value_tiles_token_dim_padded():
    device()
    t = _special_tiles()
    pad = np.zeros((16, 128), np.uint16)
    pad[: t.shape[0]] = t
    xt = torch.from_numpy(np.ascontiguousarray(pad.T).view(np.int16)).view(torch.bfloat16)
    for pow2 in (False, True):
        _check_act(xt, fg.FG_ALONG_ROWS, pow2)
        _check_w(torch.from_numpy(pad.view(np.int16)).view(torch.bfloat16), pow2)


@pytest.mark.parametrize("pow2", [False, True])
def test_every_finite_bf16_value(pow2):
    """Each finite bf16 pattern appears once, in tiles of 128 consecutive patterns (so tile max-abs
    values span the whole exponent range), and again in tiles whose max-abs is fixed at 448 * 2^j."""
    device()
    allb = np.arange(65536, dtype=np.uint32)
    finite = allb[((allb >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    n = (finite.size // 128) * 128
    a = finite[:n].reshape(-1, 128)
    rng = np.random.default_rng(3)
    b = rng.permutation(finite)[:n].reshape(-1, 128).copy()
    b[:, 0] = np.where(np.arange(b.shape[0]) % 2 == 0, 0x43E0, 0x7F00)        # 448 or 2^127 max
    x = np.concatenate([a, b])
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    _check_act(xt, fg.FG_ALONG_COLS, pow2)
    _check_act(xt[:, :128].contiguous()[: (x.shape[0] // 128) * 128], fg.FG_ALONG_ROWS, pow2)


def _amax_mantissa_rows(exponents=(0x20, 0x3F, 0x7F, 0x85, 0xC0)):
    """bf16 rows of 128 whose max-abs runs over all 128 bf16 mantissas at several exponents, with both
    signs and the max at a varying position; every other entry is smaller in magnitude, of random sign.
    In fp32-scale mode the quotient max / RN(max / 448) comes out as 448 * (1 + 2^-23) in fp32 for some of
    these mantissas, and the encoder must still give the code of 448."""
    rng = np.random.default_rng(77)
    rows = []
    for e in exponents:
        for m in range(128):
            for sign in (0, 1):
                top = (e << 7) | m
                rest = rng.integers(0, top, 127).astype(np.uint16) | (rng.integers(0, 2, 127).astype(np.uint16) << 15)
                pos = int(rng.integers(0, 128))
                rows.append(np.insert(rest, pos, np.uint16((sign << 15) | top)))
    return np.stack(rows).astype(np.uint16)


def _assert_max_code_448(q_tiles):
    """Every tile (last axis) holds a code of magnitude 448 (0x7E or 0xFE)."""
    mags = np.asarray(q_tiles) & 0x7F
    assert np.all(mags.max(axis=-1) == 0x7E), "a tile whose max-abs should encode to 448 does not"


@pytest.mark.parametrize("pow2", [False, True])
def test_quotient_at_448_every_mantissa(pow2):
    """Deterministic cover of the quotient edge above 448: 1x128 tiles along the columns and along the
    rows, both tilings from one read, and 128x128 weight blocks, each with its max-abs on every bf16
    mantissa (five exponents, both signs); bit-exact against the oracle, and in fp32-scale mode every
    tile's largest code is 448."""
    device()
    t = _amax_mantissa_rows()                                     # [1280, 128]
    x = torch.from_numpy(t.view(np.int16)).view(torch.bfloat16)
    _check_act(x, fg.FG_ALONG_COLS, pow2)
    xt = torch.from_numpy(np.ascontiguousarray(t.T).view(np.int16)).view(torch.bfloat16)   # [128, 1280]
    _check_act(xt, fg.FG_ALONG_ROWS, pow2)
    _check_both(x, pow2)
    # weight blocks: block b is 128 rows of smaller entries plus the tile's max-abs entry in its first row
    rng = np.random.default_rng(78)
    nb = t.shape[0] // 8                                          # 160 blocks, every 8th row's max-abs
    wb = np.empty((nb * 128, 128), np.uint16)
    for b in range(nb):
        top = int(np.max(t[8 * b] & 0x7FFF))
        blk = rng.integers(0, top, (128, 128)).astype(np.uint16) | (rng.integers(0, 2, (128, 128)).astype(np.uint16) << 15)
        blk[0] = t[8 * b]
        wb[b * 128:(b + 1) * 128] = blk
    _check_w(torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16), pow2)
    if not pow2:
        q, _ = fg.fg_quantize_act_1x128(to_dev(x))
        _assert_max_code_448(np_u8(q))
        qw, _ = fg.fg_quantize_w_128x128(to_dev(torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16)))
        _assert_max_code_448(np_u8(qw).reshape(nb, 128 * 128))


def test_deterministic_repeat(dsv3):
    x = to_dev(dsv3[0])
    q1, s1 = fg.fg_quantize_act_1x128(x)
    q2, s2 = fg.fg_quantize_act_1x128(x)
    assert torch.equal(q1, q2) and torch.equal(s1, s2)


# ------------------------------------------------------------------------------------------------
# Both tilings from one read (fg_quantize_act_1x128_both): bit-exact against the oracle's two tilings
# ------------------------------------------------------------------------------------------------

def _check_both(x_cpu, pow2, ld_pad=0):
    xb = bits(x_cpu)
    x = to_dev(x_cpu)
    if ld_pad:
        big = torch.zeros((x.shape[0], x.shape[1] + ld_pad), dtype=torch.bfloat16, device=x.device)
        big[:, : x.shape[1]] = x
        x = big[:, : x_cpu.shape[1]]
    qc, sc, qr, sr = fg.fg_quantize_act_1x128_both(x, pow2=pow2)
    torch.cuda.synchronize()
    for axis, q, s in ((fg.FG_ALONG_COLS, qc, sc), (fg.FG_ALONG_ROWS, qr, sr)):
        q_ref, s_ref = oracle.quantize_act_1x128(xb, axis, pow2)
        assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), f"axis {axis}: scales differ"
        bad = np.argwhere(np_u8(q) != q_ref)
        assert bad.size == 0, f"axis {axis}: {len(bad)} codes differ, first {bad[:5].tolist()}"


@pytest.mark.parametrize("pow2", [False, True])
def test_both_dsv3_activation_and_gradient(dsv3, pow2):
    x, _, dy = dsv3
    _check_both(x, pow2)
    _check_both(dy, pow2)


@pytest.mark.parametrize("rows,cols,ld_pad", [(128, 128, 0), (256, 384, 8), (384, 1024, 24)])
@pytest.mark.parametrize("pow2", [False, True])
def test_both_shapes_and_strides(rows, cols, ld_pad, pow2):
    device()
    rng = np.random.default_rng(rows * 7 + cols)
    _check_both(wl.normal_bf16(rng, (rows, cols), 1.0, outlier_channels=3, outlier_scale=40.0), pow2, ld_pad)


def test_both_special_values():
    """Special rows (zeros, signed zeros, subnormals, extremes, ties, tiny scales) placed both as rows and,
    transposed, as columns of one 256 x 128 block, so each edge case drives a row tile and a column tile."""
    device()
    t = _special_tiles()
    a = np.zeros((128, 128), np.uint16)
    a[: t.shape[0]] = t
    x = np.concatenate([a, np.ascontiguousarray(a.T)])
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    for pow2 in (False, True):
        _check_both(xt, pow2)


@pytest.mark.parametrize("pow2", [False, True])
def test_both_every_finite_bf16_value(pow2):
    device()
    allb = np.arange(65536, dtype=np.uint32)
    finite = allb[((allb >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    n = (finite.size // (128 * 128)) * 128 * 128
    x = finite[:n].reshape(-1, 128)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    _check_both(xt, pow2)


# ------------------------------------------------------------------------------------------------
# The Linear operator's two forward operands in one launch (fg_quantize_fprop_operands): X in both
# 1x128 tilings and W in 128x128 blocks, bit-exact against the oracle. Every output buffer starts filled
# with a sentinel (0x55 codes, NaN scales), so an element the launch never writes cannot pass.
# ------------------------------------------------------------------------------------------------

def _sentinel_u8(shape):
    return torch.full(shape, 0x55, dtype=torch.uint8, device="cuda")


def _sentinel_f32(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def _padded(t_cpu, ld_pad):
    t = to_dev(t_cpu)
    if not ld_pad:
        return t
    big = torch.zeros((t.shape[0], t.shape[1] + ld_pad), dtype=torch.bfloat16, device=t.device)
    big[:, : t.shape[1]] = t
    return big[:, : t_cpu.shape[1]]


def _check_fprop_operands(x_cpu, w_cpu, pow2, ld_pad=0):
    rows, k = x_cpu.shape
    n = w_cpu.shape[0]
    x, w = _padded(x_cpu, ld_pad), _padded(w_cpu, 2 * ld_pad)
    outs = (_sentinel_u8((rows, k)), _sentinel_f32((k // 128, rows)), _sentinel_u8((k, rows)),
            _sentinel_f32(((rows + 127) // 128, k)), _sentinel_u8((n, k)), _sentinel_f32(((n + 127) // 128, k // 128)))
    qc, sc, qr, sr, qw, sw = fg.fg_quantize_fprop_operands(x, w, pow2=pow2, q_cols=outs[0], scales_cols=outs[1],
                                                           q_rows=outs[2], scales_rows=outs[3], qw=outs[4], sw=outs[5])
    torch.cuda.synchronize()
    if rows:
        xb = bits(x_cpu)
        for axis, q, s in ((fg.FG_ALONG_COLS, qc, sc), (fg.FG_ALONG_ROWS, qr, sr)):
            q_ref, s_ref = oracle.quantize_act_1x128(xb, axis, pow2)
            assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), f"x axis {axis}: scales"
            bad = np.argwhere(np_u8(q) != q_ref)
            assert bad.size == 0, f"x axis {axis}: {len(bad)} codes differ, first {bad[:5].tolist()}"
    else:
        assert torch.all(qc == 0x55) and torch.all(qr == 0x55), "an empty X must not be written"
    if n:
        q_ref, s_ref = oracle.quantize_w_128x128(bits(w_cpu), pow2)
        assert np.array_equal(sw.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), "w scales differ"
        bad = np.argwhere(np_u8(qw) != q_ref)
        assert bad.size == 0, f"w: {len(bad)} codes differ, first {bad[:5].tolist()}"


@pytest.mark.parametrize("pow2", [False, True])
def test_fprop_operands_dsv3(dsv3, pow2):
    """The dense-MLP step's X [4096, 7168] and W [18432, 7168], as the step quantizes them."""
    x, w, _ = dsv3
    _check_fprop_operands(x, w, pow2)


@pytest.mark.parametrize("rows,n,k,ld_pad", [(128, 128, 128, 0), (256, 300, 384, 8), (384, 1000, 1024, 24),
                                             (0, 300, 256, 0), (256, 0, 256, 8), (128, 1, 128, 0)])
@pytest.mark.parametrize("pow2", [False, True])
def test_fprop_operands_shapes(rows, n, k, ld_pad, pow2):
    """Ragged weight rows, strided inputs, and either tensor empty (its outputs must stay untouched)."""
    device()
    rng = np.random.default_rng(rows * 131 + n * 7 + k)
    x = wl.normal_bf16(rng, (rows, k), 1.0, outlier_channels=min(3, k), outlier_scale=40.0)
    w = wl.normal_bf16(rng, (n, k), 0.02)
    _check_fprop_operands(x, w, pow2, ld_pad)


def test_fprop_operands_special_values():
    """Special rows (zeros, signed zeros, subnormals, extremes, ties, tiny scales) in X as rows and as
    columns, and in W as block rows."""
    device()
    t = _special_tiles()
    a = np.zeros((128, 128), np.uint16)
    a[: t.shape[0]] = t
    x = np.concatenate([a, np.ascontiguousarray(a.T)])
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    for pow2 in (False, True):
        _check_fprop_operands(xt, xt, pow2)
