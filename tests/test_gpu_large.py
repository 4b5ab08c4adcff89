"""GPU parity past 2^31 elements: the quantizers and the GEMM address their operands with 64-bit offsets.

Inputs are seeded on the device (torch's generator) and only the parts the checks need are copied to the
host. Each check is local, so the oracle runs on slices:
  * 1x128 tiles along the columns of X [65600, 32768] (2.15 G elements): the rows past element 2^31 and a
    sample of earlier rows, against the oracle on those rows;
  * tiles along the tokens of a [262272, 8192] tensor (2.15 G elements): sampled column bands (the last
    one's transposed codes reach past byte 2^31), against the oracle on the same column bands;
  * Fprop with X [262400, 8192] (2.15 G codes): sampled output rows against the oracle on those rows.
"""
import numpy as np
import pytest
import torch

import fp8_fine_grained_amax_amd as fg
import oracle
from tests.gpu_util import TOL_F32, bits, device, normwise, np_u8

pytestmark = pytest.mark.gpu


def _randn_bf16(shape, seed, std=1.0):
    g = torch.Generator(device=device())
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=device(), dtype=torch.float32) * std).to(torch.bfloat16)


def test_quantize_rows_past_2_31():
    rows, cols = 65600, 32768                       # 2^31 + 2.1 M elements
    x = _randn_bf16((rows, cols), 901)
    q, s = fg.fg_quantize_act_1x128(x)
    torch.cuda.synchronize()
    first_big = (1 << 31) // cols                   # first row whose elements lie past 2^31
    pick = np.concatenate([np.arange(first_big - 2, rows), np.array([0, 1, 777, 40000])])
    xb = bits(x[torch.as_tensor(pick, device=device())])
    q_o, s_o = oracle.quantize_act_1x128(xb, 0, False)
    idx = torch.as_tensor(pick, device=device())
    assert np.array_equal(np_u8(q[idx]), q_o)
    assert np.array_equal(s[:, idx].cpu().numpy().view(np.uint32), s_o.view(np.uint32))


def test_quantize_tokens_past_2_31():
    rows, cols = 262272, 8192                       # 2^31 + 1.0 M elements; codes written [cols][rows]
    x = _randn_bf16((rows, cols), 902)
    q, s = fg.fg_quantize_act_1x128(x, axis=fg.FG_ALONG_ROWS)
    torch.cuda.synchronize()
    for c0 in (0, 4096, 8192 - 64):                 # the last band's codes reach past byte 2^31
        xb = bits(x[:, c0:c0 + 64])
        q_o, s_o = oracle.quantize_act_1x128(xb, 1, False)
        assert np.array_equal(np_u8(q[c0:c0 + 64]), q_o), c0
        assert np.array_equal(s[:, c0:c0 + 64].cpu().numpy().view(np.uint32), s_o.view(np.uint32)), c0


def test_fprop_operand_past_2_31():
    M, N, K = 262400, 384, 8192                     # X codes: 2^31 + 2.1 M bytes
    x = _randn_bf16((M, K), 903)
    w = _randn_bf16((N, K), 904, std=0.02)
    xq, sx = fg.fg_quantize_act_1x128(x)
    del x
    wq, sw = fg.fg_quantize_w_128x128(w)
    y = fg.fg_fp8_gemm_fprop(xq, sx, wq, sw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    first_big = (1 << 31) // K
    pick = np.concatenate([np.arange(first_big - 3, first_big + 3), np.arange(M - 5, M), np.array([0, 12345])])
    idx = torch.as_tensor(pick, device=device())
    prom, _ = oracle.gemm_fprop(np_u8(xq[idx]), np.ascontiguousarray(sx[:, idx].cpu().numpy()), np_u8(wq),
                                sw.cpu().numpy(), want_exact=False)
    assert normwise(y[idx].cpu().numpy(), prom) <= TOL_F32
