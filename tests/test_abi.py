"""C-ABI checks that need no GPU: the library loads, exports every function include/fp8fg.h declares,
and rejects bad arguments on the host with the documented status codes before any HIP call."""
import ctypes
import os
import re

import pytest

import fp8_fine_grained_amax_amd as fg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8fg.h")

OK, INVALID, SHAPE, MISALIGNED = 0, 1, 2, 3
A16 = 1 << 20          # fake, 16-byte aligned "device" addresses: never dereferenced on these paths
A16B = 2 << 20
ODD = (1 << 20) + 4


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:fg_status|const char\*|int)\s+(fg_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fg.LIB_PATH):
        from fp8_fine_grained_amax_amd import build
        build.build()
    return fg.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) == 19, names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code, text in [(0, "ok"), (1, "invalid argument"), (2, "unsupported shape"),
                       (3, "misaligned pointer or leading dimension"), (4, "HIP runtime error")]:
        assert fg.fg_status_string(code) == text
    assert L.fg_last_hip_error() == 0


def test_quantize_act_rejections(L):
    q = L.fg_quantize_act_1x128
    assert q(A16, -1, 128, 128, 0, 0, A16, A16, None) == INVALID           # negative rows
    assert q(A16, 4, 128, 128, 2, 0, A16, A16, None) == INVALID            # bad axis
    assert q(A16, 4, 128, 128, 0, 5, A16, A16, None) == INVALID            # bad mode
    assert q(A16, 4, 128, 64, 0, 0, A16, A16, None) == INVALID             # ld < cols
    assert q(None, 4, 128, 128, 0, 0, A16, A16, None) == INVALID           # null input
    assert q(A16, 4, 100, 104, 0, 0, A16, A16, None) == SHAPE              # cols % 128 (along cols)
    assert q(A16, 100, 64, 64, 1, 0, A16, A16, None) == SHAPE              # rows % 128 (along rows)
    assert q(A16, 128, 60, 64, 1, 0, A16, A16, None) == SHAPE              # cols % 8 (along rows)
    assert q(ODD, 4, 128, 128, 0, 0, A16, A16, None) == MISALIGNED         # x not 16 B aligned
    assert q(A16, 4, 128, 132, 0, 0, A16, A16, None) == MISALIGNED         # ld % 8
    assert q(A16, 0, 128, 128, 0, 0, None, None, None) == OK               # empty: no-op


def test_quantize_both_rejections(L):
    q = L.fg_quantize_act_1x128_both
    assert q(A16, -1, 128, 128, 0, A16, A16, A16, A16, None) == INVALID     # negative rows
    assert q(A16, 128, 128, 128, 4, A16, A16, A16, A16, None) == INVALID    # bad mode
    assert q(A16, 128, 128, 64, 0, A16, A16, A16, A16, None) == INVALID     # ld < cols
    assert q(A16, 128, 128, 128, 0, A16, A16, None, A16, None) == INVALID   # null transposed codes
    assert q(A16, 100, 128, 128, 0, A16, A16, A16, A16, None) == SHAPE      # rows % 128
    assert q(A16, 128, 136, 136, 0, A16, A16, A16, A16, None) == SHAPE      # cols % 128
    assert q(A16, 128, 128, 128, 0, A16, A16, ODD, A16, None) == MISALIGNED
    assert q(A16, 0, 128, 128, 0, None, None, None, None, None) == OK        # empty: no-op


def test_quantize_fprop_operands_rejections(L):
    q = L.fg_quantize_fprop_operands
    out = (A16, A16, A16, A16, A16, A16)
    assert q(A16, -1, 128, A16, 128, 128, 128, 0, *out, None) == INVALID      # negative rows
    assert q(A16, 128, 128, A16, 128, 128, 128, 4, *out, None) == INVALID     # bad mode
    assert q(A16, 128, 64, A16, 128, 128, 128, 0, *out, None) == INVALID      # ld_x < k
    assert q(A16, 128, 128, A16, 128, 64, 128, 0, *out, None) == INVALID      # ld_w < k
    assert q(A16, 128, 128, None, 128, 128, 128, 0, *out, None) == INVALID    # null w
    assert q(A16, 100, 128, A16, 128, 128, 128, 0, *out, None) == SHAPE       # rows % 128
    assert q(A16, 128, 136, A16, 128, 136, 136, 0, *out, None) == SHAPE       # k % 128
    assert q(A16, 128, 132, A16, 128, 128, 128, 0, *out, None) == MISALIGNED  # ld_x % 8
    assert q(A16, 128, 128, ODD, 128, 128, 128, 0, *out, None) == MISALIGNED  # w not 16 B aligned
    assert q(None, 0, 128, None, 0, 128, 128, 0, *([None] * 6), None) == OK   # empty: no-op
    assert q(None, 128, 128, None, 128, 128, 0, 0, *([None] * 6), None) == OK  # k == 0: no-op


def test_quantize_w_rejections(L):
    q = L.fg_quantize_w_128x128
    assert q(A16, 128, 100, 100, 0, A16, A16, None) == SHAPE               # k % 128
    assert q(A16, 128, 128, 128, 3, A16, A16, None) == INVALID             # bad mode
    assert q(A16, 128, 128, 128, 0, ODD, A16, None) == MISALIGNED
    assert q(A16, 0, 128, 128, 0, None, None, None) == OK


def test_gemm_rejections(L):
    f = L.fg_fp8_gemm_fprop
    assert f(A16, A16, A16, A16, 128, 128, 100, A16, 0, 0, None) == SHAPE     # K % 128
    assert f(A16, A16, A16, A16, 128, 128, 128, A16, 7, 0, None) == INVALID   # bad out dtype
    assert f(A16, A16, A16, A16, 128, 128, 128, A16, 0, 9, None) == INVALID   # bad scale mode
    assert f(A16, A16, None, A16, 128, 128, 128, A16, 0, 0, None) == INVALID  # null W
    assert f(A16, A16, A16, A16, 128, 128, 128, ODD, 0, 0, None) == MISALIGNED
    assert f(None, None, None, None, 0, 128, 128, None, 0, 0, None) == OK     # empty
    fq = L.fg_fp8_gemm_fprop_quant
    assert fq(A16, A16, A16, A16, 128, 200, 128, A16, A16, 0, 0, None) == SHAPE   # N % 128 (output groups)
    assert fq(A16, A16, A16, A16, 128, 128, 100, A16, A16, 0, 0, None) == SHAPE   # K % 128
    assert fq(A16, A16, A16, A16, 128, 128, 128, A16, A16, 0, 2, None) == INVALID # bad output scale mode
    assert fq(A16, A16, A16, A16, 128, 128, 128, A16, None, 0, 0, None) == INVALID  # null output scales
    assert fq(A16, A16, A16, A16, 128, 128, 128, ODD, A16, 0, 0, None) == MISALIGNED
    assert fq(None, None, None, None, 0, 128, 128, None, None, 0, 0, None) == OK  # empty
    d = L.fg_fp8_gemm_dgrad
    assert d(A16, A16, A16, A16, 128, 200, 128, A16, 0, 0, None) == SHAPE     # N (contraction) % 128
    assert d(A16, A16, A16, A16, 128, 256, 200, A16, 0, 0, None) == SHAPE     # K % 128
    w = L.fg_fp8_gemm_wgrad
    assert w(A16, A16, A16, A16, 100, 128, 128, A16, 0, 0, None) == SHAPE     # M (tokens) % 128
    assert w(A16, A16, A16, A16, 128, 128, 130, A16, 0, 0, None) == SHAPE     # K % 4
    assert w(A16, A16, A16, ODD, 128, 128, 128, A16, 0, 0, None) == MISALIGNED  # per-row scales need 16 B
    g = L.fg_fp8_grouped_gemm
    assert g(A16, A16, A16, A16, A16B, 0, 128, 128, 128, A16, 0, 0, None) == INVALID   # G < 1
    assert g(A16, A16, A16, A16, None, 2, 128, 128, 128, A16, 0, 0, None) == INVALID   # null offsets
    assert g(A16, A16, A16, A16, A16B, 2, 128, 128, 100, A16, 0, 0, None) == SHAPE     # K % 128
    gd = L.fg_fp8_grouped_gemm_dgrad
    assert gd(A16, A16, A16, A16, A16B, 0, 128, 128, 128, A16, 0, 0, None) == INVALID  # G < 1
    assert gd(A16, A16, A16, A16, A16B, 2, 128, 100, 128, A16, 0, 0, None) == SHAPE    # N (contraction) % 128
    assert gd(A16, A16, A16, A16, A16B, 2, 128, 128, 128, ODD, 0, 0, None) == MISALIGNED
    assert gd(None, None, None, None, A16B, 2, 0, 128, 128, None, 0, 0, None) == OK    # empty
    gw = L.fg_fp8_grouped_gemm_wgrad
    assert gw(A16, A16, A16, A16, None, 2, 256, 128, 128, A16, 0, 0, None) == INVALID  # null offsets
    assert gw(A16, A16, A16, A16, A16B, 2, 200, 128, 128, A16, 0, 0, None) == SHAPE    # tokens % 128
    assert gw(A16, A16, A16, A16, A16B, 2, 256, 128, 130, A16, 0, 0, None) == SHAPE    # K % 4
    assert gw(A16, A16, A16, ODD, A16B, 2, 256, 128, 128, A16, 0, 0, None) == MISALIGNED
    assert L.fg_last_hip_error() == 0


def test_gemm_size_limits(L):
    """Contractions longer than 2^24 and Dgrad outputs wider than 2^25 would overflow the kernels' 32-bit
    operand offsets: rejected on the host, while the limits themselves pass the shape checks (the calls
    below that pass them use M == 0 or equivalent empty outputs, so nothing is launched)."""
    big, bigger = 1 << 24, (1 << 24) + 128
    f = L.fg_fp8_gemm_fprop
    assert f(A16, A16, A16, A16, 128, 128, bigger, A16, 0, 0, None) == SHAPE
    assert L.fg_fp8_gemm_fprop_quant(A16, A16, A16, A16, 128, 128, bigger, A16, A16, 0, 0, None) == SHAPE
    d = L.fg_fp8_gemm_dgrad
    assert d(A16, A16, A16, A16, 128, bigger, 128, A16, 0, 0, None) == SHAPE          # contraction N
    assert d(A16, A16, A16, A16, 128, 128, (1 << 25) + 128, A16, 0, 0, None) == SHAPE  # output width K
    w = L.fg_fp8_gemm_wgrad
    assert w(A16, A16, A16, A16, bigger, 128, 128, A16, 0, 0, None) == SHAPE          # tokens
    g = L.fg_fp8_grouped_gemm
    assert g(A16, A16, A16, A16, A16B, 2, 128, 128, bigger, A16, 0, 0, None) == SHAPE
    gd = L.fg_fp8_grouped_gemm_dgrad
    assert gd(A16, A16, A16, A16, A16B, 2, 128, bigger, 128, A16, 0, 0, None) == SHAPE
    assert gd(A16, A16, A16, A16, A16B, 2, 128, 128, (1 << 25) + 128, A16, 0, 0, None) == SHAPE
    gw = L.fg_fp8_grouped_gemm_wgrad
    assert gw(A16, A16, A16, A16, A16B, 2, bigger, 128, 128, A16, 0, 0, None) == SHAPE
    # at the limits the shape checks pass; with an empty output nothing is launched
    assert f(None, None, None, None, 0, 128, big, None, 0, 0, None) == OK
    assert w(None, None, None, None, big, 0, 128, None, 0, 0, None) == OK
    assert L.fg_last_hip_error() == 0


def test_python_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(fg.Fp8fgError):
        fg.fg_quantize_act_1x128(torch.zeros(4, 128, dtype=torch.bfloat16))


def test_per_tensor_rejections(L):
    a = L.fg_amax_bf16
    assert a(A16, 4, 124, 128, A16B, None) == SHAPE                  # cols % 8
    assert a(A16, 4, 128, 100, A16B, None) == INVALID                # ld < cols
    assert a(A16, 4, 128, 128, None, None) == INVALID                # null amax
    assert a(ODD, 4, 128, 128, A16B, None) == MISALIGNED
    assert a(None, 0, 128, 128, None, None) == OK                    # empty
    q = L.fg_quantize_per_tensor
    assert q(A16, 4, 100, 104, A16B, 1, 0, 0, A16, A16, None, None) == SHAPE       # cols % 128
    assert q(A16, 4, 128, 128, A16B, 5000, 0, 0, A16, A16, None, None) == SHAPE    # history too long
    assert q(A16, 4, 128, 128, A16B, 1, 3, 0, A16, A16, None, None) == INVALID     # bad mode
    assert q(A16, 4, 128, 128, A16B, 1, 0, 2, A16, A16, None, None) == INVALID     # bad layout
    assert q(A16, 4, 128, 128, None, 1, 0, 0, A16, A16, None, None) == INVALID     # null history
    assert q(A16, 4, 128, 128, A16B, 4, 0, 0, A16, A16, A16B + 8, None) == INVALID  # amax_out inside history
    assert q(A16, 4, 128, 128, A16B, 1, 0, 0, ODD, A16, None, None) == MISALIGNED
    assert q(None, 0, 128, 128, None, 0, 0, 0, None, None, None, None) == OK       # empty


def test_requantize_rejections(L):
    r = L.fg_requantize_1x128_to_tokens
    assert r(A16, A16, 100, 128, 0, A16, A16, None) == SHAPE            # rows % 128
    assert r(A16, A16, 128, 200, 0, A16, A16, None) == SHAPE            # cols % 128
    assert r(A16, A16, 128, 128, 7, A16, A16, None) == INVALID          # bad mode
    assert r(A16, None, 128, 128, 0, A16, A16, None) == INVALID         # null input scales
    assert r(A16, ODD, 128, 128, 0, A16, A16, None) == MISALIGNED       # input scales need 16 B
    assert r(None, None, 0, 128, 0, None, None, None) == OK             # empty


def test_e5m6_rejections(L):
    q = L.fg_quantize_e5m6_1x128
    assert q(A16, 4, 200, 200, A16, A16, None) == SHAPE                 # cols % 128
    assert q(A16, 4, 128, 100, A16, A16, None) == INVALID               # ld < cols
    assert q(A16, 4, 128, 128, None, A16, None) == INVALID              # null packed
    assert q(ODD, 4, 128, 128, A16, A16, None) == MISALIGNED
    assert q(A16, 4, 128, 132, A16, A16, None) == MISALIGNED            # ld % 8
    assert q(None, 0, 128, 128, None, None, None) == OK                 # empty
    d = L.fg_dequantize_e5m6_1x128
    assert d(A16, A16, 4, 200, A16, 200, None) == SHAPE
    assert d(A16, A16, 4, 128, A16, 100, None) == INVALID               # ld < cols
    assert d(A16, None, 4, 128, A16, 128, None) == INVALID              # null scales
    assert d(A16, A16, 4, 128, ODD, 128, None) == MISALIGNED
    assert d(None, None, 0, 128, None, 128, None) == OK


def test_limited_accum_rejections(L):
    f = L.fg_fp8_gemm_fprop_limited_accum
    assert f(A16, A16, A16, A16, 16, 16, 100, 10, A16, None) == SHAPE        # K % 128
    assert f(A16, A16, A16, A16, 16, 16, 128, 0, A16, None) == INVALID       # mantissa bits < 1
    assert f(A16, A16, A16, A16, 16, 16, 128, 24, A16, None) == INVALID      # mantissa bits > 23
    assert f(A16, A16, None, A16, 16, 16, 128, 10, A16, None) == INVALID     # null W
    assert f(A16 + 4, A16, A16, A16, 16, 16, 128, 10, A16, None) == MISALIGNED
    assert f(None, None, None, None, 0, 16, 128, 10, None, None) == OK       # empty
