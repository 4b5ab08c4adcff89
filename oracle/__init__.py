"""CPU oracle for fine-grained FP8 quantization and block-scaled GEMM — TEST INFRASTRUCTURE ONLY.

Thin numpy wrappers over oracle/oracle.c (plain C, IEEE fp32/fp64). Only tests, the package smoke check
and the benchmark's CPU-baseline leg import this module; the GPU library and its Python binding never do,
and the two share no code. See oracle.c for the definitions followed and the readings taken where the
source pages are silent.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode_many.argtypes = [P, I64, P]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_scale_from_amax.restype = ctypes.c_float
        L.oracle_scale_from_amax.argtypes = [ctypes.c_float, I]
        L.oracle_quantize_act_1x128.argtypes = [P, I64, I64, I64, I, I, P, P]
        L.oracle_quantize_w_128x128.argtypes = [P, I64, I64, I64, I, P, P]
        L.oracle_requantize_1x128_to_tokens.argtypes = [P, P, I64, I64, I, P, P]
        L.oracle_e5m6_decode.restype = ctypes.c_double
        L.oracle_e5m6_decode.argtypes = [ctypes.c_uint16]
        L.oracle_e5m6_encode.restype = ctypes.c_uint16
        L.oracle_e5m6_encode.argtypes = [ctypes.c_float]
        L.oracle_quantize_e5m6_1x128.argtypes = [P, I64, I64, I64, P, P]
        L.oracle_dequantize_e5m6_1x128.argtypes = [P, P, I64, I64, P]
        L.oracle_amax_bf16.restype = ctypes.c_float
        L.oracle_amax_bf16.argtypes = [P, I64, I64, I64]
        L.oracle_quantize_per_tensor.argtypes = [P, I64, I64, I64, P, I64, I, I, P, P]
        L.oracle_gemm_fprop.argtypes = [P, P, P, P, I64, I64, I64, P, I64, I, P, P]
        L.oracle_gemm_dgrad.argtypes = [P, P, P, P, I64, I64, I64, P, I64, I, P, P]
        L.oracle_gemm_wgrad.argtypes = [P, P, P, P, I64, I64, I64, I, P, I64, P, P]
        L.oracle_gemm_grouped.argtypes = [P, P, P, P, P, ctypes.c_int32, I64, I64, I64, P, I64, I, P, P]
        L.oracle_gemm_fprop_limited.argtypes = [P, P, P, P, I64, I64, I64, I64, I, P, I64, P]
        L.oracle_num_threads.restype = I
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(x):
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint16, "bf16 inputs are passed as their uint16 bit patterns"
    return x


def e4m3_decode(codes):
    """Decode E4M3 codes (any int array) to float64, elementwise."""
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib().oracle_e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[codes]


def e4m3_encode_many(values):
    """E4M3 codes of a float32 array (the oracle's encoder, element by element)."""
    v = np.ascontiguousarray(values, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_e4m3_encode_many(_p(v), v.size, _p(out))
    return out


def e4m3_encode_scalar(v: float) -> int:
    return int(lib().oracle_e4m3_encode(float(v)))


def f32_to_bf16_scalar(v: float) -> int:
    return int(lib().oracle_f32_to_bf16(float(v)))


def scale_from_amax(amax: float, pow2: bool) -> float:
    return float(lib().oracle_scale_from_amax(float(amax), int(pow2)))


def quantize_act_1x128(x_bits, axis: int, pow2: bool):
    """x_bits: uint16 [rows, cols] bf16 bit patterns. axis 0: tiles along columns, returns
    (q uint8 [rows, cols], scales f32 [ceil(cols/128), rows]). axis 1: tiles along rows (token dim),
    returns (q uint8 [cols, rows] transposed, scales f32 [ceil(rows/128), cols])."""
    x = _u16(x_bits)
    rows, cols = x.shape
    if axis == 0:
        q = np.empty((rows, cols), np.uint8)
        s = np.empty(((cols + 127) // 128, rows), np.float32)
    else:
        q = np.empty((cols, rows), np.uint8)
        s = np.empty(((rows + 127) // 128, cols), np.float32)
    lib().oracle_quantize_act_1x128(_p(x), rows, cols, cols, axis, int(pow2), _p(q), _p(s))
    return q, s


def quantize_w_128x128(w_bits, pow2: bool):
    """w_bits: uint16 [n, k]. Returns (q uint8 [n, k], scales f32 [ceil(n/128), ceil(k/128)])."""
    w = _u16(w_bits)
    n, k = w.shape
    q = np.empty((n, k), np.uint8)
    s = np.empty(((n + 127) // 128, (k + 127) // 128), np.float32)
    lib().oracle_quantize_w_128x128(_p(w), n, k, k, int(pow2), _p(q), _p(s))
    return q, s


def requantize_1x128_to_tokens(q, s, pow2: bool):
    """Cached 1x128 codes q uint8 [rows, cols] with scales s f32 [cols/128, rows] -> token tiles of the bf16
    activations they stand for: (q_out uint8 [cols, rows], s_out f32 [ceil(rows/128), cols])."""
    q = np.ascontiguousarray(q, np.uint8)
    s = np.ascontiguousarray(s, np.float32)
    rows, cols = q.shape
    q_out = np.empty((cols, rows), np.uint8)
    s_out = np.empty(((rows + 127) // 128, cols), np.float32)
    lib().oracle_requantize_1x128_to_tokens(_p(q), _p(s), rows, cols, int(pow2), _p(q_out), _p(s_out))
    return q_out, s_out


def e5m6_decode(codes):
    """Values of 12-bit E5M6 codes (array), float64."""
    c = np.asarray(codes, np.uint16)
    table = np.array([lib().oracle_e5m6_decode(i) for i in range(4096)], np.float64)
    return table[c & 0xFFF]


def e5m6_encode(values):
    """E5M6 codes of float32 values (array)."""
    v = np.asarray(values, np.float32).reshape(-1)
    return np.array([lib().oracle_e5m6_encode(float(f)) for f in v], np.uint16).reshape(np.shape(values))


def quantize_e5m6_1x128(x_bits):
    """bf16 bits [rows, cols] -> (packed uint8 [rows, cols * 3 / 2], scales f32 [cols/128, rows])."""
    x = _u16(x_bits)
    rows, cols = x.shape
    packed = np.empty((rows, cols * 3 // 2), np.uint8)
    s = np.empty((cols // 128, rows), np.float32)
    lib().oracle_quantize_e5m6_1x128(_p(x), rows, cols, cols, _p(packed), _p(s))
    return packed, s


def dequantize_e5m6_1x128(packed, scales):
    """bf16 bits [rows, cols] that E5M6 storage stands for."""
    packed = np.ascontiguousarray(packed, np.uint8)
    scales = np.ascontiguousarray(scales, np.float32)
    rows, cols = packed.shape[0], packed.shape[1] * 2 // 3
    y = np.empty((rows, cols), np.uint16)
    lib().oracle_dequantize_e5m6_1x128(_p(packed), _p(scales), rows, cols, _p(y))
    return y


def e5m6_unpack(packed):
    """12-bit codes [rows, cols] from packed [rows, cols * 3 / 2] (three bytes per two codes)."""
    p = np.asarray(packed, np.uint16).reshape(packed.shape[0], -1, 3)
    c0 = p[..., 0] | ((p[..., 1] & 0xF) << 8)
    c1 = (p[..., 1] >> 4) | (p[..., 2] << 4)
    return np.stack([c0, c1], axis=-1).reshape(packed.shape[0], -1)


def amax_bf16(x_bits):
    """max |x| of a uint16 bf16 matrix, as a float."""
    x = _u16(x_bits)
    rows, cols = x.shape
    return float(lib().oracle_amax_bf16(_p(x), rows, cols, cols))


def quantize_per_tensor(x_bits, hist, pow2: bool, layout: int = 0):
    """One scale for the whole matrix from the max-abs history hist (floats). layout 0: scales broadcast
    as [ceil(cols/128), rows]; layout 1: as [ceil(rows/128), ceil(cols/128)]. Returns (q, scales)."""
    x = _u16(x_bits)
    rows, cols = x.shape
    h = np.ascontiguousarray(np.asarray(hist, np.float32).reshape(-1))
    q = np.empty((rows, cols), np.uint8)
    shape = ((cols + 127) // 128, rows) if layout == 0 else ((rows + 127) // 128, (cols + 127) // 128)
    s = np.empty(shape, np.float32)
    lib().oracle_quantize_per_tensor(_p(x), rows, cols, cols, _p(h) if h.size else None, h.size, int(pow2),
                                     int(layout), _p(q), _p(s))
    return q, s


def _points(pts):
    if pts is None:
        return None, 0
    pts = np.ascontiguousarray(pts, dtype=np.int64)
    return pts, pts.size


def _outs(n, out_bf16, shape, want_exact):
    out = np.empty(n, np.uint16 if out_bf16 else np.float32)
    exact = np.empty(n, np.float64) if want_exact else None
    if shape is not None:
        out = out.reshape(shape)
        if exact is not None:
            exact = exact.reshape(shape)
    return out, exact


def gemm_fprop(xq, sx, wq, sw, out_bf16=False, pts=None, want_exact=True):
    """Y = X W^T with per-128 promotion. Returns (promoted, exact fp64). With pts (flat row-major output
    indices) only those outputs are computed, in that order; promoted is uint16 bf16 bits if out_bf16."""
    M, K = xq.shape
    N = wq.shape[0]
    pts, npts = _points(pts)
    out, exact = _outs(npts if pts is not None else M * N, out_bf16, None if pts is not None else (M, N), want_exact)
    lib().oracle_gemm_fprop(_p(np.ascontiguousarray(xq)), _p(np.ascontiguousarray(sx)), _p(np.ascontiguousarray(wq)),
                            _p(np.ascontiguousarray(sw)), M, N, K, _p(pts), npts, int(out_bf16), _p(out), _p(exact))
    return out, exact


def gemm_dgrad(dyq, sdy, wq, sw, out_bf16=False, pts=None, want_exact=True):
    """dX = dY W. dyq [M, N], sdy [N/128, M], wq [N, K], sw [N/128, ceil(K/128)]."""
    M, N = dyq.shape
    K = wq.shape[1]
    pts, npts = _points(pts)
    out, exact = _outs(npts if pts is not None else M * K, out_bf16, None if pts is not None else (M, K), want_exact)
    lib().oracle_gemm_dgrad(_p(np.ascontiguousarray(dyq)), _p(np.ascontiguousarray(sdy)), _p(np.ascontiguousarray(wq)),
                            _p(np.ascontiguousarray(sw)), M, N, K, _p(pts), npts, int(out_bf16), _p(out), _p(exact))
    return out, exact


def gemm_wgrad(dytq, sdyt, xtq, sxt, dw_init=None, pts=None, want_exact=True):
    """dW (+)= dY^T X from token-dim quantized operands. dytq [N, M], sdyt [M/128, N], xtq [K, M],
    sxt [M/128, K]. dw_init (fp32, same indexing as the outputs) turns on accumulation."""
    N, M = dytq.shape
    K = xtq.shape[0]
    pts, npts = _points(pts)
    n_out = npts if pts is not None else N * K
    if dw_init is not None:
        out = np.array(dw_init, dtype=np.float32, copy=True).reshape(-1)
        assert out.size == n_out
    else:
        out = np.empty(n_out, np.float32)
    exact = np.empty(n_out, np.float64) if want_exact else None
    lib().oracle_gemm_wgrad(_p(np.ascontiguousarray(dytq)), _p(np.ascontiguousarray(sdyt)), _p(np.ascontiguousarray(xtq)),
                            _p(np.ascontiguousarray(sxt)), M, N, K, int(dw_init is not None), _p(pts), npts,
                            _p(out), _p(exact))
    if pts is None:
        out = out.reshape(N, K)
        if exact is not None:
            exact = exact.reshape(N, K)
    return out, exact


def gemm_grouped(xq, sx, wq, sw, offsets, out_bf16=True, pts=None, want_exact=True):
    """Per group g: Y[off[g]:off[g+1]] = X[off[g]:off[g+1]] W[g]^T. wq [G, N, K], sw [G, ceil(N/128), K/128]."""
    T, K = xq.shape
    G, N, _ = wq.shape
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    pts, npts = _points(pts)
    out, exact = _outs(npts if pts is not None else T * N, out_bf16, None if pts is not None else (T, N), want_exact)
    lib().oracle_gemm_grouped(_p(np.ascontiguousarray(xq)), _p(np.ascontiguousarray(sx)), _p(np.ascontiguousarray(wq)),
                              _p(np.ascontiguousarray(sw)), _p(off), G, T, N, K, _p(pts), npts, int(out_bf16),
                              _p(out), _p(exact))
    return out, exact


def gemm_fprop_limited(xq, sx, wq, sw, chunk=32, bits=13, pts=None):
    """Fprop with a single limited-precision accumulator (no promotion): fp64 result array."""
    M, K = xq.shape
    N = wq.shape[0]
    pts, npts = _points(pts)
    out = np.empty(npts if pts is not None else M * N, np.float64)
    lib().oracle_gemm_fprop_limited(_p(np.ascontiguousarray(xq)), _p(np.ascontiguousarray(sx)), _p(np.ascontiguousarray(wq)),
                                    _p(np.ascontiguousarray(sw)), M, N, K, chunk, bits, _p(pts), npts, _p(out))
    return out if pts is not None else out.reshape(M, N)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def bf16_bits_to_f32(bits):
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
