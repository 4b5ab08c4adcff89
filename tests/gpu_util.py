"""Shared helpers for the GPU parity tests (device placement, comparisons, sampled outputs)."""
import os

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


def elementwise_large(y, ref, frac=0.01):
    """Elementwise max |y - ref| / |ref| over the entries with |ref| >= frac * max |ref|: the error metric
    reported beside the normwise gate (entries far below the largest carry no relative precision)."""
    y = np.asarray(y, np.float64).reshape(-1)
    ref = np.asarray(ref, np.float64).reshape(-1)
    big = np.abs(ref) >= frac * max(np.max(np.abs(ref)), 1e-300)
    if not np.any(big):
        return 0.0
    return float(np.max(np.abs(y[big] - ref[big]) / np.abs(ref[big])))


# (test id, output, outputs compared, normwise error, elementwise error over large entries), filled by the
# GEMM parity checks and printed in the session's terminal summary
GEMM_ERRORS = []


def record_gemm_error(what, y, ref):
    name = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0].split("::")[-1]
    GEMM_ERRORS.append((name, what, int(np.asarray(ref).size), normwise(y, ref), elementwise_large(y, ref)))


def output_tile_points(rows, cols, tile_rows, tile_cols, seed):
    """One random flat index inside every tile_rows x tile_cols block of a rows x cols output, the ragged
    edge blocks included: with 64 x 64 blocks every wave's tile of either workgroup shape is sampled, so a
    tile written to the wrong place or not at all cannot pass unseen."""
    rng = np.random.default_rng(seed)
    r0 = np.arange(0, rows, tile_rows, dtype=np.int64)
    c0 = np.arange(0, cols, tile_cols, dtype=np.int64)
    R0, C0 = np.meshgrid(r0, c0, indexing="ij")
    rr = R0 + (rng.random(R0.shape) * np.minimum(tile_rows, rows - R0)).astype(np.int64)
    cc = C0 + (rng.random(C0.shape) * np.minimum(tile_cols, cols - C0)).astype(np.int64)
    return (rr * cols + cc).reshape(-1)


def stratified_points(rows, cols, n_random, seed):
    """sample_points plus one point in every 64 x 64 output block."""
    return np.unique(np.concatenate([sample_points(rows, cols, n_random, seed),
                                     output_tile_points(rows, cols, 64, 64, seed + 1000)]))


def nan_like_out(shape, dtype):
    """An output buffer filled with NaN, so an element the kernel never writes fails the finiteness check."""
    return torch.full(shape, float("nan"), dtype=dtype, device=device())


def assert_all_written(t, what):
    bad = int((~torch.isfinite(t)).sum().item())
    assert bad == 0, f"{what}: {bad} outputs not written (still NaN) or not finite"


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
