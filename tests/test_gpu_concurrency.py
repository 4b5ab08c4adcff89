"""The library keeps no state between calls beyond per-device facts cached on first use, so calls from
several host threads on several streams at once must give the results of the same calls made one after
another. Four threads, each with its own stream and inputs, run the quantizers and the three GEMMs five
times; every output is compared bit for bit with a sequential run on the default stream.
"""
import threading

import numpy as np
import pytest
import torch

import fp8_fine_grained_amax_amd as fg
from fp8_fine_grained_amax_amd import workloads as wl
from tests.gpu_util import device, to_dev

pytestmark = pytest.mark.gpu


def _work(x, w, dy, pow2):
    xq, sx, xtq, sxt = fg.fg_quantize_act_1x128_both(x, pow2=pow2)
    wq, sw = fg.fg_quantize_w_128x128(w, pow2=pow2)
    y = fg.fg_fp8_gemm_fprop(xq, sx, wq, sw, pow2=pow2)
    dyq, sdy, dytq, sdyt = fg.fg_quantize_act_1x128_both(dy, pow2=pow2)
    dx = fg.fg_fp8_gemm_dgrad(dyq, sdy, wq, sw, pow2=pow2)
    dw = fg.fg_fp8_gemm_wgrad(dytq, sdyt, xtq, sxt, pow2=pow2)
    return [xq, sx, wq, sw, y, dx, dw]


def test_threads_and_streams_match_sequential():
    dev = device()
    rng = np.random.default_rng(91)
    cases = []
    for i in range(4):
        M, N, K = 384 + 128 * i, 512, 640
        cases.append((to_dev(wl.normal_bf16(rng, (M, K), 1.0, outlier_channels=4, outlier_scale=20.0)),
                      to_dev(wl.normal_bf16(rng, (N, K), 0.02)), to_dev(wl.normal_bf16(rng, (M, N), 1e-3)), i % 2 == 1))
    expected = [[t.clone() for t in _work(*c)] for c in cases]
    torch.cuda.synchronize()

    results, errors = [None] * len(cases), []

    def worker(i):
        try:
            stream = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(stream):
                for _ in range(5):
                    out = _work(*cases[i])
                stream.synchronize()
            results[i] = out
        except Exception as e:          # reported below, from the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i, (got, want) in enumerate(zip(results, expected)):
        for j, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"case {i}, output {j}"
