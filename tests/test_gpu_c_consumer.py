"""The C ABI used from C++ alone gives the same bits as the Python binding.

tests/c_consumer.cpp includes only include/fp8fg.h and the HIP runtime, allocates its own device buffers and
runs one training-step Linear (X and W quantized in one launch, dY in both tilings, Fprop BF16, Dgrad and
Wgrad FP32, FP32 scales) on X [256, 512], W [384, 512], dY [256, 384] from a fixed integer generator, and
checks that a malformed call is rejected. This test regenerates the same inputs, runs the same launches
through the Python binding, and compares every code, scale and output bit for bit. The binding's results
are themselves checked against the oracle by the other GPU tests.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import fp8_fine_grained_amax_amd as fg
from tests.gpu_util import device

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_consumer")
M, N, K = 256, 384, 512
MASK = (1 << 64) - 1


def bf16_inputs(seed, count, e0):
    """The consumer's generator: a 64-bit LCG; sign bit 63, exponent e0 + bits 40..42, mantissa bits 33..39."""
    out = np.empty(count, np.uint16)
    s = seed
    for i in range(count):
        s = (s * 6364136223846793005 + 1442695040888963407) & MASK
        out[i] = ((s >> 63) << 15) | ((e0 + ((s >> 40) & 7)) << 7) | ((s >> 33) & 0x7F)
    return out


def _bf16(bits, shape):
    return torch.from_numpy(bits.view(np.int16).reshape(shape).copy()).view(torch.bfloat16).cuda()


def test_c_consumer_matches_binding(tmp_path):
    device()
    assert os.path.exists(EXE), "tests/c_consumer is not built (run __graft_entry__.build())"
    out_file = tmp_path / "c_consumer.bin"
    r = subprocess.run([EXE, str(out_file)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c_consumer done" in r.stdout

    x = _bf16(bf16_inputs(1, M * K, 120), (M, K))
    w = _bf16(bf16_inputs(2, N * K, 115), (N, K))
    dy = _bf16(bf16_inputs(3, M * N, 110), (M, N))
    xq, sx, xtq, sxt, wq, sw = fg.fg_quantize_fprop_operands(x, w)
    y = fg.fg_fp8_gemm_fprop(xq, sx, wq, sw, out_dtype=torch.bfloat16)
    dyq, sdy, dytq, sdyt = fg.fg_quantize_act_1x128_both(dy)
    dx = fg.fg_fp8_gemm_dgrad(dyq, sdy, wq, sw, out_dtype=torch.float32)
    dw = fg.fg_fp8_gemm_wgrad(dytq, sdyt, xtq, sxt)
    torch.cuda.synchronize()

    blob = out_file.read_bytes()
    pos = 0
    for name, t in (("xq", xq), ("sx", sx), ("xtq", xtq), ("sxt", sxt), ("wq", wq), ("sw", sw), ("dyq", dyq),
                    ("sdy", sdy), ("dytq", dytq), ("sdyt", sdyt), ("y", y), ("dx", dx), ("dw", dw)):
        mine = t.contiguous().view(torch.uint8).cpu().numpy().ravel()
        theirs = np.frombuffer(blob, np.uint8, count=mine.size, offset=pos)
        pos += mine.size
        assert np.array_equal(mine, theirs), f"{name} differs between the C++ caller and the Python binding"
    assert pos == len(blob), "the C++ caller wrote an unexpected amount of data"
    # the inputs are ordinary finite values and the outputs must be too
    assert torch.isfinite(y.float()).all() and torch.isfinite(dx).all() and torch.isfinite(dw).all()
