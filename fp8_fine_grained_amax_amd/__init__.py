"""Fine-grained FP8 quantization and block-scaled GEMMs for MI355X (gfx950).

Thin ctypes binding over libfp8fg.so (HIP kernels + C ABI, declared in include/fp8fg.h). The Python
functions carry the C names and only marshal arguments: torch tensors provide device memory and the
current HIP stream; every step of the computation runs in the library's kernels. There is no CPU
fallback: if the library is missing or the tensors are not on a GPU, the calls raise.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8fg.so")

FG_SCALE_FP32, FG_SCALE_POW2 = 0, 1
FG_OUT_F32, FG_OUT_BF16 = 0, 1
FG_ALONG_COLS, FG_ALONG_ROWS = 0, 1
FG_LAYOUT_ACT_1x128, FG_LAYOUT_W_128x128 = 0, 1

_lib = None


class Fp8fgError(RuntimeError):
    pass


def lib():
    """Load libfp8fg.so (built in-tree by fp8_fine_grained_amax_amd/build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise Fp8fgError(f"{LIB_PATH} is not built; run fp8_fine_grained_amax_amd/build.py (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int32
        L.fg_quantize_act_1x128.argtypes = [P, I64, I64, I64, I, I, P, P, P]
        L.fg_quantize_w_128x128.argtypes = [P, I64, I64, I64, I, P, P, P]
        L.fg_quantize_act_1x128_both.argtypes = [P, I64, I64, I64, I, P, P, P, P, P]
        L.fg_quantize_fprop_operands.argtypes = [P, I64, I64, P, I64, I64, I64, I, P, P, P, P, P, P, P]
        L.fg_fp8_gemm_fprop.argtypes = [P, P, P, P, I64, I64, I64, P, I, I, P]
        L.fg_fp8_gemm_fprop_quant.argtypes = [P, P, P, P, I64, I64, I64, P, P, I, I, P]
        L.fg_fp8_gemm_dgrad.argtypes = [P, P, P, P, I64, I64, I64, P, I, I, P]
        L.fg_fp8_gemm_wgrad.argtypes = [P, P, P, P, I64, I64, I64, P, I, I, P]
        L.fg_fp8_grouped_gemm.argtypes = [P, P, P, P, P, I32, I64, I64, I64, P, I, I, P]
        L.fg_fp8_grouped_gemm_dgrad.argtypes = [P, P, P, P, P, I32, I64, I64, I64, P, I, I, P]
        L.fg_fp8_grouped_gemm_wgrad.argtypes = [P, P, P, P, P, I32, I64, I64, I64, P, I, I, P]
        L.fg_amax_bf16.argtypes = [P, I64, I64, I64, P, P]
        L.fg_fp8_gemm_fprop_limited_accum.argtypes = [P, P, P, P, I64, I64, I64, I, P, P]
        L.fg_quantize_e5m6_1x128.argtypes = [P, I64, I64, I64, P, P, P]
        L.fg_dequantize_e5m6_1x128.argtypes = [P, P, I64, I64, P, I64, P]
        L.fg_requantize_1x128_to_tokens.argtypes = [P, P, I64, I64, I, P, P, P]
        L.fg_quantize_per_tensor.argtypes = [P, I64, I64, I64, P, I64, I, I, P, P, P, P]
        for f in ("fg_quantize_act_1x128", "fg_quantize_act_1x128_both", "fg_quantize_fprop_operands",
                  "fg_quantize_w_128x128", "fg_fp8_gemm_fprop",
                  "fg_fp8_gemm_fprop_quant", "fg_fp8_gemm_dgrad", "fg_fp8_gemm_wgrad", "fg_fp8_grouped_gemm",
                  "fg_fp8_grouped_gemm_dgrad", "fg_fp8_grouped_gemm_wgrad", "fg_amax_bf16", "fg_quantize_per_tensor",
                  "fg_requantize_1x128_to_tokens", "fg_quantize_e5m6_1x128", "fg_dequantize_e5m6_1x128",
                  "fg_fp8_gemm_fprop_limited_accum"):
            getattr(L, f).restype = I
        L.fg_status_string.argtypes = [I]
        L.fg_status_string.restype = ctypes.c_char_p
        L.fg_last_hip_error.argtypes = []
        L.fg_last_hip_error.restype = I
        _lib = L
    return _lib


def fg_status_string(status: int) -> str:
    return lib().fg_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != 0:
        extra = f" (hipError {lib().fg_last_hip_error()})" if status == 4 else ""
        raise Fp8fgError(f"{what}: {fg_status_string(status)}{extra}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _gpu(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise Fp8fgError("fp8fg operates on GPU tensors only")


def _out_code(dtype):
    if dtype == torch.float32:
        return FG_OUT_F32
    if dtype == torch.bfloat16:
        return FG_OUT_BF16
    raise Fp8fgError(f"output dtype must be float32 or bfloat16, got {dtype}")


def fg_quantize_act_1x128(x, axis: int = FG_ALONG_COLS, pow2: bool = False, q=None, scales=None):
    """1x128 E4M3 quantization of a bf16 matrix x [rows, cols] (row stride may exceed cols).

    axis FG_ALONG_COLS: returns q uint8 [rows, cols], scales f32 [cols/128, rows].
    axis FG_ALONG_ROWS (token dim): returns q uint8 [cols, rows] (transposed), scales f32 [rows/128, cols].
    """
    _gpu(x)
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise Fp8fgError("x must be a 2-D bf16 tensor with unit column stride")
    rows, cols = x.shape
    if axis == FG_ALONG_COLS:
        qshape, sshape = (rows, cols), ((cols + 127) // 128, rows)
    else:
        qshape, sshape = (cols, rows), ((rows + 127) // 128, cols)
    if q is None:
        q = torch.empty(qshape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.float32, device=x.device)
    _check(lib().fg_quantize_act_1x128(_ptr(x), rows, cols, x.stride(0), int(axis),
                                       FG_SCALE_POW2 if pow2 else FG_SCALE_FP32, _ptr(q), _ptr(scales),
                                       _stream(x.device)), "fg_quantize_act_1x128")
    return q, scales


def fg_quantize_act_1x128_both(x, pow2: bool = False, q_cols=None, scales_cols=None, q_rows=None, scales_rows=None):
    """Both 1x128 tilings of a bf16 [rows, cols] matrix from one read: returns (q_cols [rows, cols],
    scales_cols [cols/128, rows], q_rows [cols, rows], scales_rows [rows/128, cols]), identical to
    fg_quantize_act_1x128 with FG_ALONG_COLS and with FG_ALONG_ROWS."""
    _gpu(x)
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise Fp8fgError("x must be a 2-D bf16 tensor with unit column stride")
    rows, cols = x.shape
    dev = x.device
    if q_cols is None:
        q_cols = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if scales_cols is None:
        scales_cols = torch.empty(((cols + 127) // 128, rows), dtype=torch.float32, device=dev)
    if q_rows is None:
        q_rows = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
    if scales_rows is None:
        scales_rows = torch.empty(((rows + 127) // 128, cols), dtype=torch.float32, device=dev)
    _check(lib().fg_quantize_act_1x128_both(_ptr(x), rows, cols, x.stride(0), FG_SCALE_POW2 if pow2 else FG_SCALE_FP32,
                                            _ptr(q_cols), _ptr(scales_cols), _ptr(q_rows), _ptr(scales_rows),
                                            _stream(dev)), "fg_quantize_act_1x128_both")
    return q_cols, scales_cols, q_rows, scales_rows


def fg_requantize_1x128_to_tokens(q_in, s_in, pow2: bool = False, q_out=None, s_out=None):
    """Token tiles from cached 1x128 FP8 tiles: q_in uint8 [rows, cols] and s_in f32 [cols/128, rows] (as
    fg_quantize_act_1x128 along columns) -> (q_out uint8 [cols, rows], s_out f32 [rows/128, cols])."""
    _gpu(q_in, s_in, q_out, s_out)
    rows, cols = q_in.shape
    if q_out is None:
        q_out = torch.empty((cols, rows), dtype=torch.uint8, device=q_in.device)
    if s_out is None:
        s_out = torch.empty((rows // 128, cols), dtype=torch.float32, device=q_in.device)
    _check(lib().fg_requantize_1x128_to_tokens(_ptr(q_in), _ptr(s_in), rows, cols, _mode(pow2), _ptr(q_out),
                                               _ptr(s_out), _stream(q_in.device)), "fg_requantize_1x128_to_tokens")
    return q_out, s_out


def fg_quantize_w_128x128(w, pow2: bool = False, q=None, scales=None):
    """128x128-block E4M3 quantization of a bf16 weight w [n, k]: q uint8 [n, k], scales f32 [ceil(n/128), k/128]."""
    _gpu(w)
    if w.dtype != torch.bfloat16 or w.dim() != 2 or w.stride(1) != 1:
        raise Fp8fgError("w must be a 2-D bf16 tensor with unit column stride")
    n, k = w.shape
    if q is None:
        q = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty(((n + 127) // 128, (k + 127) // 128), dtype=torch.float32, device=w.device)
    _check(lib().fg_quantize_w_128x128(_ptr(w), n, k, w.stride(0), FG_SCALE_POW2 if pow2 else FG_SCALE_FP32,
                                       _ptr(q), _ptr(scales), _stream(w.device)), "fg_quantize_w_128x128")
    return q, scales


def fg_quantize_fprop_operands(x, w, pow2: bool = False, q_cols=None, scales_cols=None, q_rows=None,
                               scales_rows=None, qw=None, sw=None):
    """X [rows, k] in both 1x128 tilings and W [n, k] in 128x128 blocks from one kernel launch: returns
    (q_cols, scales_cols, q_rows, scales_rows, qw, sw), identical to fg_quantize_act_1x128_both(x) followed
    by fg_quantize_w_128x128(w)."""
    _gpu(x, w)
    for t, what in ((x, "x"), (w, "w")):
        # an empty tensor is not read, whatever its strides
        if t.dtype != torch.bfloat16 or t.dim() != 2 or (t.numel() > 0 and t.stride(1) != 1):
            raise Fp8fgError(f"{what} must be a 2-D bf16 tensor with unit column stride")
    rows, k = x.shape
    n, kw = w.shape
    if kw != k:
        raise Fp8fgError(f"x and w must share the contraction width: {k} != {kw}")
    dev = x.device
    if q_cols is None:
        q_cols = torch.empty((rows, k), dtype=torch.uint8, device=dev)
    if scales_cols is None:
        scales_cols = torch.empty(((k + 127) // 128, rows), dtype=torch.float32, device=dev)
    if q_rows is None:
        q_rows = torch.empty((k, rows), dtype=torch.uint8, device=dev)
    if scales_rows is None:
        scales_rows = torch.empty(((rows + 127) // 128, k), dtype=torch.float32, device=dev)
    if qw is None:
        qw = torch.empty((n, k), dtype=torch.uint8, device=dev)
    if sw is None:
        sw = torch.empty(((n + 127) // 128, (k + 127) // 128), dtype=torch.float32, device=dev)
    _check(lib().fg_quantize_fprop_operands(_ptr(x), rows, x.stride(0), _ptr(w), n, w.stride(0), k, _mode(pow2),
                                            _ptr(q_cols), _ptr(scales_cols), _ptr(q_rows), _ptr(scales_rows), _ptr(qw),
                                            _ptr(sw), _stream(dev)), "fg_quantize_fprop_operands")
    return q_cols, scales_cols, q_rows, scales_rows, qw, sw


def _bf16_2d(x, what):
    _gpu(x)
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise Fp8fgError(f"{what} must be a 2-D bf16 tensor with unit column stride")
    return x.shape


def fg_quantize_e5m6_1x128(x, packed=None, scales=None):
    """E5M6 storage of a bf16 matrix x [rows, cols] in 1x128 tiles with power-of-2 scales: returns
    (packed uint8 [rows, cols * 3 / 2], scales f32 [cols/128, rows])."""
    rows, cols = _bf16_2d(x, "x")
    if packed is None:
        packed = torch.empty((rows, cols * 3 // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((cols // 128, rows), dtype=torch.float32, device=x.device)
    _gpu(packed, scales)
    _check(lib().fg_quantize_e5m6_1x128(_ptr(x), rows, cols, x.stride(0), _ptr(packed), _ptr(scales),
                                        _stream(x.device)), "fg_quantize_e5m6_1x128")
    return packed, scales


def fg_dequantize_e5m6_1x128(packed, scales, y=None):
    """bf16 [rows, cols] from E5M6 storage (packed uint8 [rows, cols * 3 / 2], scales f32 [cols/128, rows])."""
    _gpu(packed, scales, y)
    rows = packed.shape[0]
    cols = packed.shape[1] * 2 // 3
    if y is None:
        y = torch.empty((rows, cols), dtype=torch.bfloat16, device=packed.device)
    _check(lib().fg_dequantize_e5m6_1x128(_ptr(packed), _ptr(scales), rows, cols, _ptr(y), y.stride(0),
                                          _stream(packed.device)), "fg_dequantize_e5m6_1x128")
    return y


def fg_amax_bf16(x, amax=None):
    """max |x| of a bf16 matrix, folded into the device float amax (a new zero-filled one if None)."""
    rows, cols = _bf16_2d(x, "x")
    if amax is None:
        amax = torch.zeros((1,), dtype=torch.float32, device=x.device)
    _gpu(amax)
    _check(lib().fg_amax_bf16(_ptr(x), rows, cols, x.stride(0), _ptr(amax), _stream(x.device)), "fg_amax_bf16")
    return amax


def fg_quantize_per_tensor(x, amax_hist, pow2: bool = False, layout: int = FG_LAYOUT_ACT_1x128, q=None, scales=None,
                           amax_out=None):
    """One E4M3 scale for the whole bf16 matrix x [rows, cols] from the device max-abs history amax_hist
    (1-D float32). Returns (q uint8 [rows, cols], scales) with scales broadcast in the 1x128 activation
    layout [cols/128, rows] or the 128x128 weight layout [ceil(rows/128), cols/128]."""
    rows, cols = _bf16_2d(x, "x")
    _gpu(amax_hist, amax_out)
    if amax_hist.dtype != torch.float32 or amax_hist.dim() != 1 or not amax_hist.is_contiguous():
        raise Fp8fgError("amax_hist must be a contiguous 1-D float32 tensor")
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if scales is None:
        shape = (cols // 128, rows) if layout == FG_LAYOUT_ACT_1x128 else ((rows + 127) // 128, cols // 128)
        scales = torch.empty(shape, dtype=torch.float32, device=x.device)
    _check(lib().fg_quantize_per_tensor(_ptr(x), rows, cols, x.stride(0), _ptr(amax_hist), amax_hist.numel(),
                                        _mode(pow2), layout, _ptr(q), _ptr(scales), _ptr(amax_out),
                                        _stream(x.device)), "fg_quantize_per_tensor")
    return q, scales


def _mode(pow2):
    return FG_SCALE_POW2 if pow2 else FG_SCALE_FP32


def fg_fp8_gemm_fprop(xq, sx, wq, sw, out_dtype=torch.bfloat16, y=None, pow2: bool = False):
    """Y [M, N] = X [M, K] . W [N, K]^T from E4M3 codes and their scales (pow2: all scales are powers of two)."""
    _gpu(xq, sx, wq, sw, y)
    M, K = xq.shape
    N = wq.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=xq.device)
    _check(lib().fg_fp8_gemm_fprop(_ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), M, N, K, _ptr(y), _out_code(y.dtype),
                                   _mode(pow2), _stream(xq.device)), "fg_fp8_gemm_fprop")
    return y


def fg_fp8_gemm_fprop_quant(xq, sx, wq, sw, yq=None, sy=None, pow2: bool = False, out_pow2: bool = False):
    """Fprop whose BF16 output leaves the GEMM already quantized 1x128 along its columns: returns
    (yq u8 [M, N], sy f32 [N/128, M]), equal to fg_quantize_act_1x128 of fg_fp8_gemm_fprop's BF16 Y."""
    _gpu(xq, sx, wq, sw, yq, sy)
    M, K = xq.shape
    N = wq.shape[0]
    if yq is None:
        yq = torch.empty((M, N), dtype=torch.uint8, device=xq.device)
    if sy is None:
        sy = torch.empty((N // 128, M), dtype=torch.float32, device=xq.device)
    _check(lib().fg_fp8_gemm_fprop_quant(_ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), M, N, K, _ptr(yq), _ptr(sy),
                                         _mode(pow2), _mode(out_pow2), _stream(xq.device)), "fg_fp8_gemm_fprop_quant")
    return yq, sy


def fg_fp8_gemm_fprop_limited_accum(xq, sx, wq, sw, mantissa_bits: int, y=None):
    """Accuracy study: Fprop without FP32 promotion, 32-element matrix-core chunks added to an FP32
    accumulator truncated to `mantissa_bits` explicit mantissa bits after every addition. fp32 [M, N]."""
    _gpu(xq, sx, wq, sw, y)
    M, K = xq.shape
    N = wq.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    _check(lib().fg_fp8_gemm_fprop_limited_accum(_ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), M, N, K, int(mantissa_bits),
                                                 _ptr(y), _stream(xq.device)), "fg_fp8_gemm_fprop_limited_accum")
    return y


def fg_fp8_gemm_dgrad(dyq, sdy, wq, sw, out_dtype=torch.float32, dx=None, pow2: bool = False):
    """dX [M, K] = dY [M, N] . W [N, K], contracting over N, with W's codes and 128x128 block scales."""
    _gpu(dyq, sdy, wq, sw, dx)
    M, N = dyq.shape
    K = wq.shape[1]
    if dx is None:
        dx = torch.empty((M, K), dtype=out_dtype, device=dyq.device)
    _check(lib().fg_fp8_gemm_dgrad(_ptr(dyq), _ptr(sdy), _ptr(wq), _ptr(sw), M, N, K, _ptr(dx), _out_code(dx.dtype),
                                   _mode(pow2), _stream(dyq.device)), "fg_fp8_gemm_dgrad")
    return dx


def fg_fp8_gemm_wgrad(dytq, sdyt, xtq, sxt, dw=None, accumulate: bool = False, pow2: bool = False):
    """dW [N, K] (+)= dY^T . X from token-dim quantized dYt [N, M] and Xt [K, M]; fp32 output."""
    _gpu(dytq, sdyt, xtq, sxt, dw)
    N, M = dytq.shape
    K = xtq.shape[0]
    if dw is None:
        if accumulate:
            raise Fp8fgError("accumulate needs an existing dw")
        dw = torch.empty((N, K), dtype=torch.float32, device=dytq.device)
    _check(lib().fg_fp8_gemm_wgrad(_ptr(dytq), _ptr(sdyt), _ptr(xtq), _ptr(sxt), M, N, K, _ptr(dw), int(bool(accumulate)),
                                   _mode(pow2), _stream(dytq.device)), "fg_fp8_gemm_wgrad")
    return dw


def fg_fp8_grouped_gemm(xq, sx, wq, sw, offsets, out_dtype=torch.bfloat16, y=None, pow2: bool = False):
    """Per group g: Y[off[g]:off[g+1]] = X[off[g]:off[g+1]] . W[g]^T. offsets: device int32 [G+1]."""
    _gpu(xq, sx, wq, sw, offsets, y)
    if offsets.dtype != torch.int32:
        raise Fp8fgError("offsets must be int32")
    T, K = xq.shape
    G, N, _ = wq.shape
    if y is None:
        y = torch.empty((T, N), dtype=out_dtype, device=xq.device)
    _check(lib().fg_fp8_grouped_gemm(_ptr(xq), _ptr(sx), _ptr(wq), _ptr(sw), _ptr(offsets), G, T, N, K, _ptr(y),
                                     _out_code(y.dtype), _mode(pow2), _stream(xq.device)), "fg_fp8_grouped_gemm")
    return y


def fg_fp8_grouped_gemm_dgrad(dyq, sdy, wq, sw, offsets, out_dtype=torch.float32, dx=None, pow2: bool = False):
    """Per group g: dX[off[g]:off[g+1]] = dY[off[g]:off[g+1]] . W[g]. dyq [T, N], wq [G, N, K]; offsets: device int32."""
    _gpu(dyq, sdy, wq, sw, offsets, dx)
    if offsets.dtype != torch.int32:
        raise Fp8fgError("offsets must be int32")
    T, N = dyq.shape
    G, _, K = wq.shape
    if dx is None:
        dx = torch.empty((T, K), dtype=out_dtype, device=dyq.device)
    _check(lib().fg_fp8_grouped_gemm_dgrad(_ptr(dyq), _ptr(sdy), _ptr(wq), _ptr(sw), _ptr(offsets), G, T, N, K, _ptr(dx),
                                           _out_code(dx.dtype), _mode(pow2), _stream(dyq.device)),
           "fg_fp8_grouped_gemm_dgrad")
    return dx


def fg_fp8_grouped_gemm_wgrad(dytq, sdyt, xtq, sxt, offsets, dw=None, accumulate: bool = False, pow2: bool = False):
    """Per group g: dW[g] (+)= dY[tokens of g]^T . X[tokens of g] from token-dim quantized dYt [N, T] and
    Xt [K, T]; every offset a multiple of 128. Returns dw f32 [G, N, K]."""
    _gpu(dytq, sdyt, xtq, sxt, offsets, dw)
    if offsets.dtype != torch.int32:
        raise Fp8fgError("offsets must be int32")
    N, T = dytq.shape
    K = xtq.shape[0]
    G = offsets.numel() - 1
    if dw is None:
        if accumulate:
            raise Fp8fgError("accumulate needs an existing dw")
        dw = torch.empty((G, N, K), dtype=torch.float32, device=dytq.device)
    _check(lib().fg_fp8_grouped_gemm_wgrad(_ptr(dytq), _ptr(sdyt), _ptr(xtq), _ptr(sxt), _ptr(offsets), G, T, N, K,
                                           _ptr(dw), int(bool(accumulate)), _mode(pow2), _stream(dytq.device)),
           "fg_fp8_grouped_gemm_wgrad")
    return dw
