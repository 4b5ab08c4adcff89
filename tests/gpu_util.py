"""Shared helpers for the GPU parity tests (device placement, comparisons, sampled outputs)."""
import numpy as np
import torch

import fp8_fine_grained_amax_amd as fg
import oracle
from fp8_fine_grained_amax_amd import workloads as wl

# Tolerances on the normwise max relative error max|y - y_ref| / max|y_ref| against the oracle's
# promoted result: 1e-3 for FP32 outputs, 1e-2 for BF16 outputs (both sides rounded to BF16).
TOL_F32 = 1e-3
TOL_BF16 = 1e-2


def device():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    fg.lib()                                  # fail loudly if the native library is missing
    return torch.device("cuda:0")


def to_dev(t):
    return t.to(device())


def np_u8(t):
    return t.detach().cpu().numpy()


def np_f32(t):
    return t.detach().float().cpu().numpy() if t.dtype != torch.bfloat16 else \
        oracle.bf16_bits_to_f32(wl.bf16_bits(t))


def bits(t):
    return wl.bf16_bits(t)


def normwise(y, ref):
    y = np.asarray(y, np.float64).reshape(-1)
    ref = np.asarray(ref, np.float64).reshape(-1)
    return float(np.max(np.abs(y - ref)) / max(np.max(np.abs(ref)), 1e-300))


def bf16_bits_to_f64(b):
    return oracle.bf16_bits_to_f32(b).astype(np.float64)


def sample_points(rows, cols, n, seed):
    """Sampled flat output indices: the four corners, the last row and column, and random points."""
    rng = np.random.default_rng(seed)
    fixed = [0, cols - 1, (rows - 1) * cols, rows * cols - 1]
    fixed += [(rows - 1) * cols + c for c in rng.integers(0, cols, 16)]
    fixed += [r * cols + cols - 1 for r in rng.integers(0, rows, 16)]
    pts = np.concatenate([np.array(fixed, np.int64), rng.integers(0, rows * cols, n, dtype=np.int64)])
    return np.unique(pts)
