"""Seeded synthetic inputs for the fine-grained FP8 workloads.

This module only draws random numbers and casts them to bfloat16 (round-to-nearest-even, torch's CPU
cast). It holds none of the quantization or GEMM arithmetic; the GPU path and the CPU oracle both take
their inputs from here and from nowhere else. Values are drawn with numpy's PCG64 in float32, outlier
channels are multiplied in before the cast, and the bf16 bits are what both sides see.

Shapes and distributions follow the workloads of the fine-grained FP8 pages: a DeepSeek-V3-like dense
MLP Linear (hidden 7168, intermediate 18432, 4096 tokens), its backward pair, an accumulation-precision
stress test at K = 4096 / 16384, and one GPU's share of an MoE layer (8 experts, hidden 7168, expert
intermediate 2048; [W4] passage on the MoE layer: 256 routed experts with intermediate 2048, 8 active per
token; [W5]: each GPU hosts 8 experts).
"""
from dataclasses import dataclass

import numpy as np
import torch


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """float32 numpy -> bf16 CPU tensor (RNE)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> numpy uint16 bit patterns."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def normal_bf16(rng, shape, std, outlier_channels=0, outlier_scale=1.0):
    a = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    if outlier_channels:
        cols = rng.choice(shape[-1], outlier_channels, replace=False)
        a[..., cols] *= np.float32(outlier_scale)
    return to_bf16(a)


def uniform_bf16(rng, shape, lo=0.0, hi=1.0):
    return to_bf16(rng.uniform(lo, hi, size=shape).astype(np.float32))


# ---------------------------------------------------------------------------------------------------
# Workload definitions
# ---------------------------------------------------------------------------------------------------

@dataclass
class LinearShape:
    M: int   # tokens
    N: int   # output channels
    K: int   # input channels


TINY = LinearShape(128, 256, 512)
DSV3_MLP = LinearShape(4096, 18432, 7168)


def tiny_fprop(seed=1001):
    """X [128,512] ~N(0,1) with 4 outlier channels x50; W [256,512] ~N(0,0.02)."""
    rng = np.random.default_rng(seed)
    x = normal_bf16(rng, (TINY.M, TINY.K), 1.0, outlier_channels=4, outlier_scale=50.0)
    w = normal_bf16(rng, (TINY.N, TINY.K), 0.02)
    return x, w


def dsv3_fprop(seed=1002, shape=DSV3_MLP):
    """X [4096,7168] ~N(0,1) with round(1% of 7168) = 72 outlier channels x20; W [18432,7168] ~N(0,0.006)."""
    rng = np.random.default_rng(seed)
    x = normal_bf16(rng, (shape.M, shape.K), 1.0, outlier_channels=int(round(0.01 * shape.K)), outlier_scale=20.0)
    w = normal_bf16(rng, (shape.N, shape.K), 0.006)
    return x, w


def dsv3_backward_dy(seed=1003, shape=DSV3_MLP):
    """dY [4096,18432] ~N(0,1e-3) (the backward pair reuses the forward X and W)."""
    rng = np.random.default_rng(seed)
    return normal_bf16(rng, (shape.M, shape.N), 1e-3)


def accumulation_stress(K, seed=1004, M=1024, N=1024):
    """X [1024,K], W [1024,K] ~U(0,1): all-positive, so block sums grow with K."""
    rng = np.random.default_rng(seed + K)
    x = uniform_bf16(rng, (M, K))
    w = uniform_bf16(rng, (N, K))
    return x, w


MOE_EXPERTS = 8
MOE_HIDDEN = 7168
MOE_INTER = 2048
MOE_TOKENS = 8192
MOE_TOPK = 8


def moe_rows(seed=1005, experts=MOE_EXPERTS, assignments=MOE_TOKENS * MOE_TOPK, skew=1.1):
    """Rows per local expert: the 8192 x top-8 = 65536 (token, expert) assignments spread over the 8
    local experts by a multinomial draw with Zipf(1.1) popularity p_e ~ (e+1)^-1.1."""
    rng = np.random.default_rng(seed)
    p = (np.arange(1, experts + 1, dtype=np.float64)) ** (-skew)
    p /= p.sum()
    rows = rng.multinomial(assignments, p).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    return rows, offsets


def moe_inputs(seed=1005, rows_scale=1.0, hidden=MOE_HIDDEN, inter=MOE_INTER, experts=MOE_EXPERTS):
    """Grouped up-projection input X [sum R, hidden], down-projection input H [sum R, inter] (independent
    draw), W_up [E, inter, hidden], W_down [E, hidden, inter]. rows_scale < 1 shrinks the token count
    (same skew) for small parity cases."""
    assignments = int(round(MOE_TOKENS * MOE_TOPK * rows_scale))
    rows, offsets = moe_rows(seed, experts, assignments)
    T = int(offsets[-1])
    rng = np.random.default_rng(seed + 1)
    x = normal_bf16(rng, (T, hidden), 1.0)
    h = normal_bf16(rng, (T, inter), 1.0)
    w_up = normal_bf16(rng, (experts, inter, hidden), 0.006)
    w_down = normal_bf16(rng, (experts, hidden, inter), 0.006)
    return dict(rows=rows, offsets=offsets, x=x, h=h, w_up=w_up, w_down=w_down)


def moe_backward_inputs(seed=1006, rows_scale=1.0, hidden=MOE_HIDDEN, inter=MOE_INTER, experts=MOE_EXPERTS, pad=128):
    """The up-projection's backward on one GPU's expert share, in a routed layout whose expert segments are
    padded with zero rows to multiples of `pad` tokens (so 1x128 token tiles never straddle two experts):
    X [T, hidden] ~N(0, 1), the output gradient dY [T, inter] ~N(0, 1e-3), W_up [E, inter, hidden]
    ~N(0, 0.006), and the padded offsets [E+1]. Same Zipf(1.1) routing skew as moe_rows."""
    assignments = int(round(MOE_TOKENS * MOE_TOPK * rows_scale))
    rows, _ = moe_rows(seed, experts, assignments)
    padded = ((rows + pad - 1) // pad) * pad
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    T = int(offsets[-1])
    rng = np.random.default_rng(seed + 1)
    x = normal_bf16(rng, (T, hidden), 1.0)
    dy = normal_bf16(rng, (T, inter), 1e-3)
    keep = np.zeros(T, bool)
    for e in range(experts):
        keep[offsets[e]: offsets[e] + rows[e]] = True
    x[torch.from_numpy(~keep)] = 0
    dy[torch.from_numpy(~keep)] = 0
    w_up = normal_bf16(rng, (experts, inter, hidden), 0.006)
    return dict(rows=rows, offsets=offsets, x=x, dy=dy, w_up=w_up)
