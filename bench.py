"""Benchmark: fine-grained FP8 Linear training pass on one MI355X.

One step = the whole hot path over one batch of the DeepSeek-V3-like dense MLP Linear
(X [4096, 7168], W [18432, 7168], dY [4096, 18432], seeded synthetic bf16):
  forward : quantize X in both 1x128 tilings (along channels for Fprop, along tokens for Wgrad, one read)
            and W (128x128 blocks), both in one launch; Fprop Y = X W^T (BF16 out)
  backward: quantize dY in both tilings (one read), Dgrad dX = dY W (FP32 out), Wgrad dW = dY^T X (FP32 out)
`value` is the FP8 GEMM throughput of the whole step (3 x 2MNK FLOP over the step's wall time), with
all inputs resident in HBM when the timed region starts. Per-kernel times come from HIP events on the
stream the kernels run on.

Also reported, beside the headline: the same step with the other scale mode, with X's and W's quantizers
as two launches, and with one quantizer launch per tiling ("variants"), per-kernel roofline fractions, cold-cache quantize bandwidth (a 1 GiB
read between launches defeats the 256 MB Infinity Cache), the Fprop that quantizes its own output
against Fprop + quantizer, per-tensor (current and delayed) scaling against the 1x128 tiles, the grouped
MoE GEMMs on one GPU's expert share, the tiny and accumulation-stress Fprop shapes, Fprop and Dgrad
over whole rounds of output tiles against the step's partly filled last round, the vendor's
per-tensor FP8 GEMM at the Fprop shape, and the CPU oracle timed on a bounded sample of the workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--pow2] [--no-moe] [--no-cpu] [--no-cold]
       [--no-vendor] [--no-fused-epilogue] [--no-per-tensor] [--no-small] [--no-overlap] [--calib-copy]

The headline uses fp32 scales (amax/448); --pow2 makes power-of-2 scales the headline.
"""
import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 GEMM TFLOPS (% of dense FP8 peak) + quantize GB/s, 1 MI355X"
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense FP8 MFMA (no sparsity)
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def code_text(src):
    """Source text without its comments and with whitespace runs collapsed: what the compiler sees."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_hash():
    """Identifies the kernels' code (comments and layout excluded): the HBM counters in
    profiles/traffic_counters.json are used only for the code they were taken on."""
    h = hashlib.sha256()
    for f in ("gemm.hip", "quant.hip", "common.h"):
        h.update(code_text(open(os.path.join(ROOT, "fp8_fine_grained_amax_amd", "csrc", f)).read()).encode())
    return h.hexdigest()[:16]


def quant_bytes(rows, cols):
    """Algorithmic HBM bytes of a 1x128 / 128x128 quantization: 2 B in + 1 B out per element,
    4 B per scale (one per 128 or per 16384 elements)."""
    return rows * cols * 3 + rows * cols // 128 * 4


def quant_both_bytes(rows, cols):
    """Both tilings from one read: 2 B in + 2 x 1 B out per element, two scales per 128 elements."""
    return rows * cols * 4 + 2 * (rows * cols // 128) * 4


def quant_w_bytes(n, k):
    return n * k * 3 + (n // 128) * (k // 128) * 4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-moe", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-cold", action="store_true")
    ap.add_argument("--no-vendor", action="store_true")
    ap.add_argument("--no-fused-epilogue", action="store_true")
    ap.add_argument("--no-per-tensor", action="store_true")
    ap.add_argument("--no-small", action="store_true", help="skip the tiny, accumulation-stress and tile-round timings")
    ap.add_argument("--no-overlap", action="store_true",
                    help="skip the two-stream schedule (a profile's per-kernel means then hold sequential launches only)")
    ap.add_argument("--pow2", action="store_true", help="power-of-2 scales (quantizers round scales up to 2^k; "
                    "the GEMMs then apply them in the matrix core)")
    ap.add_argument("--calib-copy", action="store_true", help="only run a 512 MiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    dev = torch.device("cuda:0")
    if args.calib_copy:
        n = 512 << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "launches": 5}))
        return

    import fp8_fine_grained_amax_amd as fg
    from fp8_fine_grained_amax_amd import workloads as wl

    fg.lib()
    stream = torch.cuda.current_stream(dev)
    shape = wl.DSV3_MLP
    M, N, K = shape.M, shape.N, shape.K

    t_gen = time.time()
    x_c, w_c = wl.dsv3_fprop()
    dy_c = wl.dsv3_backward_dy()
    x, w, dy = x_c.to(dev), w_c.to(dev), dy_c.to(dev)
    gen_s = time.time() - t_gen
    print(f"[bench] inputs ready ({gen_s:.1f}s): X {tuple(x.shape)} W {tuple(w.shape)} dY {tuple(dy.shape)}",
          file=sys.stderr, flush=True)

    u8, f32 = torch.uint8, torch.float32
    bufs = dict(
        xq=torch.empty((M, K), dtype=u8, device=dev), sx=torch.empty((K // 128, M), dtype=f32, device=dev),
        wq=torch.empty((N, K), dtype=u8, device=dev), sw=torch.empty((N // 128, K // 128), dtype=f32, device=dev),
        y=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
        dyq=torch.empty((M, N), dtype=u8, device=dev), sdy=torch.empty((N // 128, M), dtype=f32, device=dev),
        dx=torch.empty((M, K), dtype=f32, device=dev),
        dytq=torch.empty((N, M), dtype=u8, device=dev), sdyt=torch.empty((M // 128, N), dtype=f32, device=dev),
        xtq=torch.empty((K, M), dtype=u8, device=dev), sxt=torch.empty((M // 128, K), dtype=f32, device=dev),
        dw=torch.empty((N, K), dtype=f32, device=dev),
    )
    B = bufs

    def make_ops(pow2, quant="batched"):
        """The step's launches. "fused": X and dY are read once each and quantized in both tilings (rows for
        Fprop/Dgrad, tokens for Wgrad) by fg_quantize_act_1x128_both, W by fg_quantize_w_128x128; "batched":
        the same, with X's and W's quantization in one launch (fg_quantize_fprop_operands); "separate": each
        tiling has its own launch."""
        if quant == "batched":
            return [
                ("quant_xw", lambda: fg.fg_quantize_fprop_operands(x, w, pow2=pow2, q_cols=B["xq"], scales_cols=B["sx"],
                                                                   q_rows=B["xtq"], scales_rows=B["sxt"], qw=B["wq"],
                                                                   sw=B["sw"]),
                 "hbm", quant_both_bytes(M, K) + quant_w_bytes(N, K)),
                ("fprop", lambda: fg.fg_fp8_gemm_fprop(B["xq"], B["sx"], B["wq"], B["sw"], y=B["y"], pow2=pow2),
                 "mfma", 2.0 * M * N * K),
                ("quant_dy_both", lambda: fg.fg_quantize_act_1x128_both(dy, pow2=pow2, q_cols=B["dyq"], scales_cols=B["sdy"],
                                                                        q_rows=B["dytq"], scales_rows=B["sdyt"]),
                 "hbm", quant_both_bytes(M, N)),
                ("dgrad", lambda: fg.fg_fp8_gemm_dgrad(B["dyq"], B["sdy"], B["wq"], B["sw"], dx=B["dx"], pow2=pow2),
                 "mfma", 2.0 * M * N * K),
                ("wgrad", lambda: fg.fg_fp8_gemm_wgrad(B["dytq"], B["sdyt"], B["xtq"], B["sxt"], dw=B["dw"], pow2=pow2),
                 "mfma", 2.0 * M * N * K),
            ]
        if quant == "fused":
            return [
                ("quant_x_both", lambda: fg.fg_quantize_act_1x128_both(x, pow2=pow2, q_cols=B["xq"], scales_cols=B["sx"],
                                                                       q_rows=B["xtq"], scales_rows=B["sxt"]),
                 "hbm", quant_both_bytes(M, K)),
                ("quant_w_128x128", lambda: fg.fg_quantize_w_128x128(w, q=B["wq"], scales=B["sw"], pow2=pow2),
                 "hbm", quant_w_bytes(N, K)),
                ("fprop", lambda: fg.fg_fp8_gemm_fprop(B["xq"], B["sx"], B["wq"], B["sw"], y=B["y"], pow2=pow2),
                 "mfma", 2.0 * M * N * K),
                ("quant_dy_both", lambda: fg.fg_quantize_act_1x128_both(dy, pow2=pow2, q_cols=B["dyq"], scales_cols=B["sdy"],
                                                                        q_rows=B["dytq"], scales_rows=B["sdyt"]),
                 "hbm", quant_both_bytes(M, N)),
                ("dgrad", lambda: fg.fg_fp8_gemm_dgrad(B["dyq"], B["sdy"], B["wq"], B["sw"], dx=B["dx"], pow2=pow2),
                 "mfma", 2.0 * M * N * K),
                ("wgrad", lambda: fg.fg_fp8_gemm_wgrad(B["dytq"], B["sdyt"], B["xtq"], B["sxt"], dw=B["dw"], pow2=pow2),
                 "mfma", 2.0 * M * N * K),
            ]
        return [
            ("quant_x_rowwise", lambda: fg.fg_quantize_act_1x128(x, q=B["xq"], scales=B["sx"], pow2=pow2),
             "hbm", quant_bytes(M, K)),
            ("quant_w_128x128", lambda: fg.fg_quantize_w_128x128(w, q=B["wq"], scales=B["sw"], pow2=pow2),
             "hbm", quant_w_bytes(N, K)),
            ("fprop", lambda: fg.fg_fp8_gemm_fprop(B["xq"], B["sx"], B["wq"], B["sw"], y=B["y"], pow2=pow2),
             "mfma", 2.0 * M * N * K),
            ("quant_dy_rowwise", lambda: fg.fg_quantize_act_1x128(dy, q=B["dyq"], scales=B["sdy"], pow2=pow2),
             "hbm", quant_bytes(M, N)),
            ("dgrad", lambda: fg.fg_fp8_gemm_dgrad(B["dyq"], B["sdy"], B["wq"], B["sw"], dx=B["dx"], pow2=pow2),
             "mfma", 2.0 * M * N * K),
            ("quant_dy_tokendim", lambda: fg.fg_quantize_act_1x128(dy, axis=fg.FG_ALONG_ROWS, q=B["dytq"],
                                                                   scales=B["sdyt"], pow2=pow2),
             "hbm", quant_bytes(M, N)),
            ("quant_x_tokendim", lambda: fg.fg_quantize_act_1x128(x, axis=fg.FG_ALONG_ROWS, q=B["xtq"],
                                                                  scales=B["sxt"], pow2=pow2),
             "hbm", quant_bytes(M, K)),
            ("wgrad", lambda: fg.fg_fp8_gemm_wgrad(B["dytq"], B["sdyt"], B["xtq"], B["sxt"], dw=B["dw"], pow2=pow2),
             "mfma", 2.0 * M * N * K),
        ]

    def run_step(ops, events=None):
        for i, (_, fn, _, _) in enumerate(ops):
            if events is not None:
                events[i][0].record(stream)
            fn()
            if events is not None:
                events[i][1].record(stream)

    def measure(ops, steps, warmup, tag):
        """W untimed steps, then exactly `steps` timed steps between two device synchronisations (the step
        time); then `steps` more with HIP events recorded on the kernels' own stream around every launch
        (the per-kernel times; the events are kept out of the step time)."""
        for _ in range(warmup):
            run_step(ops)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            run_step(ops)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ops]
              for _ in range(steps)]
        for s_ in range(steps):
            run_step(ops, ev[s_])
        torch.cuda.synchronize()
        per = {name: float(np.mean([ev[s_][i][0].elapsed_time(ev[s_][i][1]) for s_ in range(steps)]))
               for i, (name, _, _, _) in enumerate(ops)}
        print(f"[bench] {tag}: timed {steps} steps after {warmup} warmup: {ms:.3f} ms/step", file=sys.stderr,
              flush=True)
        return ms, per

    def measure_graph(ops, steps, warmup, tag):
        """The same step captured once in a HIP graph and replayed: W untimed replays, then exactly `steps`
        timed replays between two device synchronisations."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_step(ops)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        print(f"[bench] {tag} (HIP graph): timed {steps} replays after {warmup} warmup: {ms:.3f} ms/step",
              file=sys.stderr, flush=True)
        return g, ms

    POW2 = bool(args.pow2)
    QUANT_DESC = {"batched": "batched quantizers", "fused": "fused quantizers", "separate": "separate quantizers"}
    # Variants of the same step on the same buffers, reported beside the headline: the other scale mode, X's
    # and W's quantizers as two launches, and one launch per tiling. They run before the headline, each with
    # its own W warmup and K timed steps. A freshly started process's first ~50 steps ran 2-3% slower than
    # the steady state on MI355X (with 5 warmup steps the timed steps fell inside that transient; with 50 or
    # more they did not, whatever the number of timed steps); the headline reports the steady state of a
    # training loop, so it is measured last.
    variants = {}
    same_mode = {}                                  # variants in the headline's scale mode: their launches
    for pw, qu in ((POW2, "separate"), (not POW2, "separate"), (POW2, "fused"), (not POW2, "fused"),
                   (not POW2, "batched")):
        vops = make_ops(pw, qu)
        vms, vper = measure(vops, args.steps, args.warmup, ("pow2" if pw else "fp32") + " scales, " + QUANT_DESC[qu])
        variants[("pow2" if pw else "fp32") + "_" + qu] = (vops, vms, vper)
        if pw == POW2:
            same_mode[qu] = (vops, vper)
    ops = make_ops(POW2, "batched")
    ms_eager, per_kernel_ms = measure(ops, args.steps, args.warmup,
                                      ("pow2" if POW2 else "fp32") + " scales, batched quantizers")
    # Two more schedules of the same kernels; each one's outputs must equal the sequential step's bit for bit
    # before its time counts:
    #  - overlapped: a second stream (default priority) runs Wgrad beside Dgrad (independent kernels: Wgrad's
    #    tiles fill Dgrad's last, partial round of workgroups);
    #  - the sequential step captured once as a HIP graph and replayed.
    side = torch.cuda.Stream(device=dev)
    by_name = {name: fn for name, fn, _, _ in ops}

    def run_step_overlap():
        main = torch.cuda.current_stream(dev)
        by_name["quant_xw"]()
        by_name["fprop"]()
        by_name["quant_dy_both"]()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            by_name["wgrad"]()
        by_name["dgrad"]()
        main.wait_stream(side)                      # the next step's X quantizer overwrites what Wgrad reads

    def timed(fn, steps, warmup, tag):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        print(f"[bench] {tag}: timed {steps} steps after {warmup} warmup: {ms:.3f} ms/step", file=sys.stderr, flush=True)
        return ms

    outs = ("y", "dx", "dw", "xq", "sx", "xtq", "sxt", "wq", "sw", "dyq", "sdy", "dytq", "sdyt")
    run_step(ops)
    torch.cuda.synchronize()
    eager_out = {k: B[k].clone() for k in outs}

    def same_as_eager():
        torch.cuda.synchronize()
        ok = all(torch.equal(B[k].view(torch.uint8), eager_out[k].view(torch.uint8)) for k in outs)
        for k in outs:
            B[k].zero_()
        return ok

    for k in outs:
        B[k].zero_()
    ms_overlap, overlap_ok = None, None
    if not args.no_overlap:
        ms_overlap = timed(run_step_overlap, args.steps, args.warmup, ("pow2" if POW2 else "fp32") + " scales, overlapped")
        overlap_ok = same_as_eager()
    graph, ms_graph = measure_graph(ops, args.steps, args.warmup, ("pow2" if POW2 else "fp32") + " scales, batched quantizers")
    graph_ok = same_as_eager()
    del eager_out, graph
    schedules = {"eager": ms_eager}
    if overlap_ok:
        schedules["overlapped"] = ms_overlap
    if graph_ok:
        schedules["hip_graph"] = ms_graph
    launch_mode = min(schedules, key=schedules.get)
    ms_per_step = schedules[launch_mode]
    # every quantizer launch of the headline's scale mode, once by name, with its in-step time
    quant_ops = {}
    for vops, vper in [(ops, per_kernel_ms)] + [same_mode[q] for q in ("fused", "separate")]:
        for o in vops:
            if o[2] == "hbm" and o[0] not in quant_ops:
                quant_ops[o[0]] = o
                per_kernel_ms.setdefault(o[0], vper[o[0]])

    gemm_flop = 3 * 2.0 * M * N * K
    value = gemm_flop / (ms_per_step * 1e-3) / 1e12

    kernels = {}
    for name, _, bound, work in [o for o in ops if o[2] == "mfma"] + list(quant_ops.values()):
        ms = per_kernel_ms[name]
        if bound == "mfma":
            ach = work / (ms * 1e-3) / 1e12
            kernels[name] = {"ms": round(ms, 4), "TFLOP/s": round(ach, 1), "frac_fp8_peak": round(ach / PEAK_FP8_TFLOPS, 4)}
        else:
            ach = work / (ms * 1e-3) / 1e9
            kernels[name] = {"ms": round(ms, 4), "GB/s": round(ach, 1), "frac_hbm_peak": round(ach / PEAK_HBM_GBPS, 4)}

    # Cold-cache quantize bandwidth: read 1 GiB before each launch (outside the timed event pair) so the
    # 256 MB Infinity Cache and the L2s hold none of the input. The scrub only reads: a written scrub
    # would leave dirty lines whose write-back the measured kernel would pay for.
    cold = {}
    if not args.no_cold:
        scrub = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        sink = torch.empty((), dtype=torch.int32, device=dev)
        for name, fn, bound, work in quant_ops.values():
            times = []
            for _ in range(7):
                torch.amax(scrub, dim=0, out=sink)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            ms = float(np.median(times))
            gbps = work / (ms * 1e-3) / 1e9
            cold[name] = {"ms": round(ms, 4), "GB/s": round(gbps, 1), "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4)}
        # Reference: plain contiguous device copies moving the same total bytes as the X- and dY-sized
        # quantizers (3 B per element: 1.5 B read + 1.5 B written here), timed the same cold way: what a
        # bandwidth-bound kernel of that size reaches on this GPU.
        for cname, n_el in (("copy_like_quant_x", M * K), ("copy_like_quant_dy", M * N)):
            src = torch.empty(3 * n_el // 2, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            times = []
            for _ in range(7):
                torch.amax(scrub, dim=0, out=sink)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                dst.copy_(src)
                e1.record(stream)
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            ms = float(np.median(times))
            gbps = 3 * n_el / (ms * 1e-3) / 1e9
            cold[cname] = {"ms": round(ms, 4), "GB/s": round(gbps, 1), "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4)}
            del src, dst
        del scrub
        print("[bench] cold-cache quantize timings done", file=sys.stderr, flush=True)

    # The small configurations (parity cases, timed for completeness): the tiny Fprop X [128,512] . W [256,512]^T
    # and the accumulation-stress Fprop X [1024,K] . W [1024,K]^T, K = 4096 and 16384, fp32 scales, FP32 out.
    # Each launch is event-timed alone (5 untimed launches, then the median and minimum of 20); at these
    # sizes the kernels are launch-bound, so the fractions of peak are small by construction.
    small = None
    if not args.no_small:
        def event_ms(fn, warm=5, iters=20):
            for _ in range(warm):
                fn()
            ts = []
            for _ in range(iters):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            return float(np.median(ts)), float(np.min(ts))

        small = {}
        cases = [("tiny_fprop_128x256x512", wl.tiny_fprop())]
        cases += [(f"accumulation_stress_1024x1024x{k}", wl.accumulation_stress(k)) for k in (4096, 16384)]
        for cname, (xs, ws) in cases:
            xd, wd = xs.to(dev), ws.to(dev)
            mm, nn, kk = xd.shape[0], wd.shape[0], xd.shape[1]
            xq_s, sx_s = fg.fg_quantize_act_1x128(xd)
            wq_s, sw_s = fg.fg_quantize_w_128x128(wd)
            y_s = torch.empty((mm, nn), dtype=torch.float32, device=dev)
            entry = {}
            for kname, fn, work, bound in (
                    ("quant_x_rowwise", lambda: fg.fg_quantize_act_1x128(xd, q=xq_s, scales=sx_s), quant_bytes(mm, kk), "hbm"),
                    ("quant_w_128x128", lambda: fg.fg_quantize_w_128x128(wd, q=wq_s, scales=sw_s), quant_w_bytes(nn, kk), "hbm"),
                    ("fprop_f32", lambda: fg.fg_fp8_gemm_fprop(xq_s, sx_s, wq_s, sw_s, out_dtype=torch.float32, y=y_s),
                     2.0 * mm * nn * kk, "mfma")):
                med, mn = event_ms(fn)
                if bound == "hbm":
                    rate = work / (med * 1e-3) / 1e9
                    entry[kname] = {"us": round(med * 1e3, 2), "min_us": round(mn * 1e3, 2), "GB/s": round(rate, 1),
                                    "frac_hbm_peak": round(rate / PEAK_HBM_GBPS, 4)}
                else:
                    rate = work / (med * 1e-3) / 1e12
                    entry[kname] = {"us": round(med * 1e3, 2), "min_us": round(mn * 1e3, 2), "TFLOP/s": round(rate, 2),
                                    "frac_fp8_peak": round(rate / PEAK_FP8_TFLOPS, 4)}
            small[cname] = entry
            del xd, wd, xq_s, sx_s, wq_s, sw_s, y_s
        print("[bench] small-configuration timings done", file=sys.stderr, flush=True)

    # Fprop whose BF16 output is wanted as 1x128 FP8 tiles (the next layer's input): the GEMM writing BF16
    # and a quantizer reading it back, against the GEMM quantizing in its epilogue (same codes and scales).
    fused_epi = None
    if not args.no_fused_epilogue:
        ops[0][1]()
        ops[1][1]()                             # X and W codes of the headline scale mode
        yq = torch.empty((M, N), dtype=u8, device=dev)
        sy = torch.empty((N // 128, M), dtype=f32, device=dev)
        two = [("fprop_bf16", lambda: fg.fg_fp8_gemm_fprop(B["xq"], B["sx"], B["wq"], B["sw"], y=B["y"], pow2=POW2),
                "mfma", 2.0 * M * N * K),
               ("quant_y_rowwise", lambda: fg.fg_quantize_act_1x128(B["y"], q=yq, scales=sy, pow2=POW2),
                "hbm", quant_bytes(M, N))]
        one = [("fprop_quant", lambda: fg.fg_fp8_gemm_fprop_quant(B["xq"], B["sx"], B["wq"], B["sw"], yq=yq, sy=sy,
                                                                 pow2=POW2, out_pow2=POW2),
                "mfma", 2.0 * M * N * K)]
        ms2, per2 = measure(two, args.steps, args.warmup, "Fprop then quantize its output")
        ms1, per1 = measure(one, args.steps, args.warmup, "Fprop quantizing in its epilogue")
        fused_epi = {"separate_ms": round(ms2, 4), "separate_kernel_ms": {k: round(v, 4) for k, v in per2.items()},
                     "fused_ms": round(ms1, 4), "fused_kernel_ms": round(per1["fprop_quant"], 4),
                     "fused_TFLOP/s": round(2.0 * M * N * K / (per1["fprop_quant"] * 1e-3) / 1e12, 1),
                     "speedup": round(ms2 / ms1, 3)}
        del yq, sy

    # Contrast baseline: per-tensor scaling of X and dY. Current scaling needs the tensor's max-abs first
    # (a second read of the input); delayed scaling takes it from a history and records the new one in
    # the same pass. Timed beside the 1x128 quantizer of the same tensor.
    per_tensor = None
    if not args.no_per_tensor:
        per_tensor = {}
        hist = torch.zeros((16,), dtype=f32, device=dev)
        hist[0] = 1.0
        for tname, t, (rows, cols), qb, sb in (("x", x, (M, K), B["xq"], B["sx"]), ("dy", dy, (M, N), B["dyq"], B["sdy"])):
            cur = torch.zeros((1,), dtype=f32, device=dev)
            rec = torch.zeros((1,), dtype=f32, device=dev)
            seq = [("amax", lambda: (cur.zero_(), fg.fg_amax_bf16(t, amax=cur)), "hbm", rows * cols * 2),
                   ("quant_current", lambda: fg.fg_quantize_per_tensor(t, cur, q=qb, scales=sb), "hbm",
                    quant_bytes(rows, cols))]
            dl = [("quant_delayed", lambda: (rec.zero_(), fg.fg_quantize_per_tensor(t, hist, q=qb, scales=sb, amax_out=rec)), "hbm",
                   quant_bytes(rows, cols))]
            tl = [("quant_1x128", lambda: fg.fg_quantize_act_1x128(t, q=qb, scales=sb), "hbm", quant_bytes(rows, cols))]
            ms_c, per_c = measure(seq, args.steps, args.warmup, f"per-tensor current scaling of {tname}")
            ms_d, _ = measure(dl, args.steps, args.warmup, f"per-tensor delayed scaling of {tname}")
            ms_t, _ = measure(tl, args.steps, args.warmup, f"1x128 quantization of {tname}")
            per_tensor[tname] = {"shape": [rows, cols], "current_ms": round(ms_c, 4),
                                 "current_kernel_ms": {k: round(v, 4) for k, v in per_c.items()},
                                 "delayed_ms": round(ms_d, 4), "tiles_1x128_ms": round(ms_t, 4)}

    # Token tiles for Wgrad from activations cached as 1x128 FP8 tiles (read codes, dequantize, transpose,
    # re-quantize) against quantizing the bf16 activations along the tokens directly.
    requant = None
    if not args.no_per_tensor:
        requant = {}
        for tname, t, (rows, cols), qb, sb, qtb, stb in (("x", x, (M, K), B["xq"], B["sx"], B["xtq"], B["sxt"]),
                                                          ("dy", dy, (M, N), B["dyq"], B["sdy"], B["dytq"], B["sdyt"])):
            fg.fg_quantize_act_1x128(t, q=qb, scales=sb, pow2=POW2)
            rq = [("requant", lambda: fg.fg_requantize_1x128_to_tokens(qb, sb, pow2=POW2, q_out=qtb, s_out=stb), "hbm", 2 * rows * cols + 2 * rows * cols // 128 * 4)]
            ms_r, _ = measure(rq, args.steps, args.warmup, f"re-quantization of cached {tname} into token tiles")
            dr = [("direct", lambda: fg.fg_quantize_act_1x128(t, axis=fg.FG_ALONG_ROWS, q=qtb, scales=stb, pow2=POW2),
                   "hbm", quant_bytes(rows, cols))]
            ms_d, _ = measure(dr, args.steps, args.warmup, f"token tiles of {tname} from bf16")
            gbps = (2 * rows * cols + 2 * rows * cols // 128 * 4) / (ms_r * 1e-3) / 1e9
            requant[tname] = {"shape": [rows, cols], "requant_ms": round(ms_r, 4), "requant_GB/s": round(gbps, 1),
                              "from_bf16_ms": round(ms_d, 4)}

    # E5M6 storage of a cached activation (X): 2 B read + 1.5 B written per value to store, the reverse
    # to load it back as bf16.
    e5m6 = None
    if not args.no_per_tensor:
        pk = torch.empty((M, K * 3 // 2), dtype=u8, device=dev)
        sk = torch.empty((K // 128, M), dtype=f32, device=dev)
        yb = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        nbytes = M * K * 2 + M * K * 3 // 2 + M * K // 128 * 4
        st = [("store", lambda: fg.fg_quantize_e5m6_1x128(x, packed=pk, scales=sk), "hbm", nbytes)]
        ld_ = [("load", lambda: fg.fg_dequantize_e5m6_1x128(pk, sk, y=yb), "hbm", nbytes)]
        ms_s, _ = measure(st, args.steps, args.warmup, "E5M6 storage of X")
        ms_l, _ = measure(ld_, args.steps, args.warmup, "E5M6 load of X")
        e5m6 = {"shape": [M, K], "store_ms": round(ms_s, 4), "store_GB/s": round(nbytes / (ms_s * 1e-3) / 1e9, 1),
                "load_ms": round(ms_l, 4), "load_GB/s": round(nbytes / (ms_l * 1e-3) / 1e9, 1)}
        del pk, sk, yb

    # Grouped MoE GEMM (one GPU's expert share): up-projection then down-projection, BF16 out.
    def back_to_back_ms(fn, warm=3, groups=5, per_group=10):
        """Time per launch of `fn` launched back to back, as in a training step: `warm` untimed launches,
        then `groups` groups of `per_group` launches between two events on the kernels' stream; the median
        group's time per launch. (A launch timed alone after the device has idled runs several percent
        slower than in a stream of work.)"""
        for _ in range(warm):
            fn()
        times = []
        for _ in range(groups):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(per_group):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / per_group)
        return float(np.median(times))

    # Whole and partial rounds of output tiles. On 256x256 tiles (forced here) the step's Fprop is 1152
    # tiles on 256 compute units (4.5 rounds) and its Dgrad 448 (1.75 rounds); the same kernels over
    # N = 16384 output columns (Fprop, 4 rounds) and K = 4096 (Dgrad, 1 round) show what the last, partly
    # filled round costs. The library's own choice for the step's Fprop, 1024 tiles of 256x288 (4 rounds),
    # is timed beside them.
    tile_rounds = None
    if not args.no_small:
        tile_rounds = {}
        Nw, Kw = 16384, 4096
        ncu = torch.cuda.get_device_properties(dev).multi_processor_count
        w_k = w[:, :Kw].contiguous()
        wkq = torch.empty((N, Kw), dtype=u8, device=dev)
        wks = torch.empty((N // 128, Kw // 128), dtype=f32, device=dev)
        y_w = torch.empty((M, Nw), dtype=torch.bfloat16, device=dev)
        dx_w = torch.empty((M, Kw), dtype=f32, device=dev)
        for mode, pw in (("fp32", False), ("pow2", True)):
            fg.fg_quantize_fprop_operands(x, w, pow2=pw, q_cols=B["xq"], scales_cols=B["sx"], q_rows=B["xtq"],
                                          scales_rows=B["sxt"], qw=B["wq"], sw=B["sw"])
            fg.fg_quantize_act_1x128(dy, q=B["dyq"], scales=B["sdy"], pow2=pw)
            fg.fg_quantize_w_128x128(w_k, q=wkq, scales=wks, pow2=pw)
            wq_w, sw_w = B["wq"][:Nw], B["sw"][:Nw // 128]
            res = {}
            tile_env = os.environ.pop("FG_GEMM_TILE", None)
            os.environ["FG_GEMM_TILE"] = "256x256"
            for name, fn, flop, tiles in [
                ("fprop_N18432", lambda: fg.fg_fp8_gemm_fprop(B["xq"], B["sx"], B["wq"], B["sw"], y=B["y"], pow2=pw),
                 2.0 * M * N * K, (M // 256) * (N // 256)),
                ("fprop_N16384", lambda: fg.fg_fp8_gemm_fprop(B["xq"], B["sx"], wq_w, sw_w, y=y_w, pow2=pw),
                 2.0 * M * Nw * K, (M // 256) * (Nw // 256)),
                ("dgrad_K7168", lambda: fg.fg_fp8_gemm_dgrad(B["dyq"], B["sdy"], B["wq"], B["sw"], dx=B["dx"], pow2=pw),
                 2.0 * M * N * K, (M // 256) * (K // 256)),
                ("dgrad_K4096", lambda: fg.fg_fp8_gemm_dgrad(B["dyq"], B["sdy"], wkq, wks, dx=dx_w, pow2=pw),
                 2.0 * M * N * Kw, (M // 256) * (Kw // 256)),
            ]:
                ms = back_to_back_ms(fn)
                ach = flop / (ms * 1e-3) / 1e12
                res[name] = {"ms": round(ms, 4), "TFLOP/s": round(ach, 1), "frac_fp8_peak": round(ach / PEAK_FP8_TFLOPS, 4),
                             "tile_rounds": round(tiles / ncu, 3), "tile": "256x256"}
            os.environ["FG_GEMM_TILE"] = "256x288"
            ms = back_to_back_ms(lambda: fg.fg_fp8_gemm_fprop(B["xq"], B["sx"], B["wq"], B["sw"], y=B["y"], pow2=pw))
            del os.environ["FG_GEMM_TILE"]
            if tile_env is not None:
                os.environ["FG_GEMM_TILE"] = tile_env
            ach = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            res["fprop_N18432_256x288"] = {"ms": round(ms, 4), "TFLOP/s": round(ach, 1),
                                           "frac_fp8_peak": round(ach / PEAK_FP8_TFLOPS, 4),
                                           "tile_rounds": round((M // 256) * (N // 288) / ncu, 3), "tile": "256x288"}
            tile_rounds[mode] = res
        del w_k, wkq, wks, y_w, dx_w
        print("[bench] tile-round timings done", file=sys.stderr, flush=True)

    moe = None
    if not args.no_moe:
        del x, w, dy, bufs, B
        d = wl.moe_inputs()
        T = int(d["offsets"][-1])
        E, I, H = wl.MOE_EXPERTS, wl.MOE_INTER, wl.MOE_HIDDEN
        xm, hm = d["x"].to(dev), d["h"].to(dev)
        wu, wd = d["w_up"].to(dev), d["w_down"].to(dev)
        off = torch.from_numpy(d["offsets"]).to(dev)
        xq, sx = fg.fg_quantize_act_1x128(xm, pow2=POW2)
        hq, sh = fg.fg_quantize_act_1x128(hm, pow2=POW2)
        wuq = torch.empty((E, I, H), dtype=u8, device=dev)
        wus = torch.empty((E, I // 128, H // 128), dtype=f32, device=dev)
        wdq = torch.empty((E, H, I), dtype=u8, device=dev)
        wds = torch.empty((E, H // 128, I // 128), dtype=f32, device=dev)
        for e in range(E):
            fg.fg_quantize_w_128x128(wu[e], q=wuq[e], scales=wus[e], pow2=POW2)
            fg.fg_quantize_w_128x128(wd[e], q=wdq[e], scales=wds[e], pow2=POW2)
        yu = torch.empty((T, I), dtype=torch.bfloat16, device=dev)
        yd = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        res = {}
        # The experts' weights are quantized in one launch each: 128x128 blocks never straddle two experts
        # (2048 and 7168 are multiples of 128), so W_up [8][2048][7168] quantized as one [16384, 7168] matrix
        # gives exactly the per-expert codes and scales, in the [E][N/128][K/128] layout.
        wu2, wuq2, wus2 = wu.view(E * I, H), wuq.view(E * I, H), wus.view(E * I // 128, H // 128)
        wd2, wdq2, wds2 = wd.view(E * H, I), wdq.view(E * H, I), wds.view(E * H // 128, I // 128)
        for name, fn, flop in [
            ("grouped_up", lambda: fg.fg_fp8_grouped_gemm(xq, sx, wuq, wus, off, y=yu, pow2=POW2), 2.0 * T * I * H),
            ("grouped_down", lambda: fg.fg_fp8_grouped_gemm(hq, sh, wdq, wds, off, y=yd, pow2=POW2), 2.0 * T * I * H),
            ("quant_moe_x_rowwise", lambda: fg.fg_quantize_act_1x128(xm, q=xq, scales=sx, pow2=POW2), ("act", T, H)),
            ("quant_moe_h_rowwise", lambda: fg.fg_quantize_act_1x128(hm, q=hq, scales=sh, pow2=POW2), ("act", T, I)),
            ("quant_moe_w_up", lambda: fg.fg_quantize_w_128x128(wu2, q=wuq2, scales=wus2, pow2=POW2), ("w", E * I, H)),
            ("quant_moe_w_down", lambda: fg.fg_quantize_w_128x128(wd2, q=wdq2, scales=wds2, pow2=POW2), ("w", E * H, I)),
        ]:
            ms = back_to_back_ms(fn)
            if not isinstance(flop, tuple):
                ach = flop / (ms * 1e-3) / 1e12
                res[name] = {"ms": round(ms, 4), "TFLOP/s": round(ach, 1), "frac_fp8_peak": round(ach / PEAK_FP8_TFLOPS, 4)}
            else:
                kind, rows_, cols_ = flop
                nbytes = quant_bytes(rows_, cols_) if kind == "act" else quant_w_bytes(rows_, cols_)
                gbps = nbytes / (ms * 1e-3) / 1e9
                res[name] = {"ms": round(ms, 4), "GB/s": round(gbps, 1), "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
                             "bytes": nbytes}
        moe = {"workload": "moe_grouped_8experts_65536rows_hidden7168_inter2048", "rows_per_expert": d["rows"].tolist(), **res}
        del xm, hm, wu, wd, xq, hq, wdq, wds, yu, yd, d, wu2, wuq2, wus2, wd2, wdq2, wds2

        # The up-projection's backward on the same expert share (routed rows padded per expert to 128
        # tokens): grouped Dgrad dX = dY . W_up[e] and grouped Wgrad dW_up[e] = dY^T X over each expert's
        # tokens, after one fused quantization of dY and X (both tilings). FLOP count over the real rows.
        b = wl.moe_backward_inputs()
        Tp = int(b["offsets"][-1])
        Treal = int(b["rows"].sum())
        xb, dyb = b["x"].to(dev), b["dy"].to(dev)
        offb = torch.from_numpy(b["offsets"]).to(dev)
        xq2, sx2, xtq2, sxt2 = fg.fg_quantize_act_1x128_both(xb, pow2=POW2)
        dyq2, sdy2, dytq2, sdyt2 = fg.fg_quantize_act_1x128_both(dyb, pow2=POW2)
        dxb = torch.empty((Tp, H), dtype=f32, device=dev)
        dxb16 = torch.empty((Tp, H), dtype=torch.bfloat16, device=dev)
        dwb = torch.empty((E, I, H), dtype=f32, device=dev)
        for name, fn, flop in [
            ("grouped_dgrad_up", lambda: fg.fg_fp8_grouped_gemm_dgrad(dyq2, sdy2, wuq, wus, offb, dx=dxb, pow2=POW2),
             2.0 * Treal * I * H),
            ("grouped_dgrad_up_bf16_out", lambda: fg.fg_fp8_grouped_gemm_dgrad(dyq2, sdy2, wuq, wus, offb, dx=dxb16,
                                                                               pow2=POW2),
             2.0 * Treal * I * H),
            ("grouped_wgrad_up", lambda: fg.fg_fp8_grouped_gemm_wgrad(dytq2, sdyt2, xtq2, sxt2, offb, dw=dwb, pow2=POW2),
             2.0 * Treal * I * H),
        ]:
            ms = back_to_back_ms(fn)
            ach = flop / (ms * 1e-3) / 1e12
            moe[name] = {"ms": round(ms, 4), "TFLOP/s": round(ach, 1), "frac_fp8_peak": round(ach / PEAK_FP8_TFLOPS, 4)}
        moe["backward_padded_rows"] = Tp
        print("[bench] grouped MoE timings done", file=sys.stderr, flush=True)

    # Roofline of the dominant (longest) GEMM kernel of the step.
    gemm_names = [n for n, _, b, _ in ops if b == "mfma"]
    dom = max(gemm_names, key=lambda n: per_kernel_ms[n])
    ach = 2.0 * M * N * K / (per_kernel_ms[dom] * 1e-3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            tr = json.load(open(TRAFFIC_FILE))
            if tr.get("kernel_source_hash") == kernel_source_hash() and dom in tr.get("bytes_per_launch", {}):
                traffic = tr["bytes_per_launch"][dom]
        except (OSError, ValueError):
            traffic = None
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_FP8_TFLOPS, 4), "traffic": traffic}

    # Context, not part of the path: the vendor library's FP8 GEMM (hipBLASLt through torch._scaled_mm, one
    # scale per tensor, no fine-grained scaling or promotion) at the Fprop shape, same E4M3 format, BF16 out.
    vendor = None
    if not args.no_vendor:
        vendor = vendor_reference(M, N, K, dev)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(kernels)

    qnames = [n for n, _, b, _ in ops if b == "hbm"]
    qbytes = sum(wk for n, _, b, wk in ops if b == "hbm")
    qms = sum(per_kernel_ms[n] for n in qnames)
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": "dsv3_dense_mlp_linear_fwd_bwd", "M_tokens": M, "N_out": N, "K_in": K,
                   "tiles": "1x128 activations, 128x128 weights", "scale_mode": "pow2" if POW2 else "fp32",
                   "quantizers": "batched: X (both tilings, read once) and W in one launch; dY both tilings from one read",
                   "accumulate": "fp32, promoted every 128 K",
                   "fprop_out": "bf16", "dgrad_out": "f32", "wgrad_out": "f32", "launch": launch_mode},
        "step_ms": {"eager": round(ms_eager, 4), "overlapped": None if ms_overlap is None else round(ms_overlap, 4),
                    "overlapped_matches_eager": overlap_ok,
                    "hip_graph": round(ms_graph, 4), "hip_graph_matches_eager": graph_ok},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "quantize_GBps_in_step": round(qbytes / (qms * 1e-3) / 1e9, 1),
        "kernels": kernels,
        "variants": {k: {"ms_per_step": round(vms, 4), "value": round(gemm_flop / (vms * 1e-3) / 1e12, 2),
                         "gemm_TFLOP/s": {n: round(2.0 * M * N * K / (vper[n] * 1e-3) / 1e12, 1)
                                          for n, _, b, _ in vops if b == "mfma"},
                         "kernel_ms": {n: round(v, 4) for n, v in vper.items()}}
                     for k, (vops, vms, vper) in variants.items()},
        "quantize_cold_cache": cold,
        "small_configs": small,
        "vendor_fp8_gemm_reference": vendor,
        "moe_grouped": moe,
        "fprop_output_quantized": fused_epi,
        "tile_rounds": tile_rounds,
        "per_tensor_contrast": per_tensor,
        "requantize_tokens": requant,
        "e5m6_storage": e5m6,
        "device": {"name": torch.cuda.get_device_name(dev),
                   "compute_units": torch.cuda.get_device_properties(dev).multi_processor_count,
                   "hip": torch.version.hip, "torch": torch.__version__},
        "seeds": {"dense_mlp_x_w": 1002, "dense_mlp_dy": 1003, "moe_forward": 1005, "moe_backward": 1006},
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(out))


def vendor_reference(M, N, K, dev):
    """hipBLASLt FP8 GEMM (torch._scaled_mm, per-tensor scales) on seeded N(0,1) E4M3 operands of the Fprop
    shape: the throughput a plain FP8 GEMM reaches on this GPU, for context."""
    import torch
    try:
        g = torch.Generator(device=dev)
        g.manual_seed(7)
        a = torch.randn((M, K), device=dev, generator=g).to(torch.float8_e4m3fn)
        b = torch.randn((N, K), device=dev, generator=g).to(torch.float8_e4m3fn)
        one = torch.tensor(1.0, device=dev)
        run = lambda: torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            run()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 20
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        return {"what": "torch._scaled_mm (hipBLASLt) E4M3 x E4M3 -> BF16, per-tensor scales",
                "shape": [M, N, K], "ms": round(ms, 4), "TFLOP/s": round(tf, 1),
                "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4)}
    except Exception as ex:                       # not available in this torch build
        return {"error": repr(ex)[:200]}


def cpu_baseline(gpu_kernels=None, budget_s=24.0):
    """The oracle as it stands, timed beside each GPU kernel of the step on the host's cores (OpenMP over
    all of them, within about `budget_s` seconds of CPU work in total):
      - the quantizers on the full tensors of the step (X both tilings, W 128x128 blocks, dY both tilings;
        the oracle has no fused kernel, so "both tilings" is its two single-tiling passes), in GB/s of the
        same algorithmic bytes the GPU rate uses;
      - Fprop, Dgrad and Wgrad on sampled outputs of the full-size GEMMs (each sample a full-depth promoted
        dot product), in TFLOP/s.
    `value` is the oracle's GEMM rate over the three sampled GEMMs together, in the unit of the headline;
    per_op gives each op's rate, the GPU kernel's rate from the same run, and their ratio."""
    import numpy as np
    import oracle
    from fp8_fine_grained_amax_amd import workloads as wl

    shape = wl.DSV3_MLP
    M, N, K = shape.M, shape.N, shape.K
    per_op = {}
    t_start = time.perf_counter()

    def timed(fn):
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t

    # quantizers: the step's own bf16 inputs
    x, w = wl.dsv3_fprop()
    dy = wl.dsv3_backward_dy()
    xb, wb, dyb = wl.bf16_bits(x), wl.bf16_bits(w), wl.bf16_bits(dy)
    del x, w, dy
    for name, fn, nbytes in (
            ("quant_x_both", lambda: (oracle.quantize_act_1x128(xb, 0, False), oracle.quantize_act_1x128(xb, 1, False)),
             quant_both_bytes(M, K)),
            ("quant_w_128x128", lambda: oracle.quantize_w_128x128(wb, False), quant_w_bytes(N, K)),
            ("quant_dy_both", lambda: (oracle.quantize_act_1x128(dyb, 0, False), oracle.quantize_act_1x128(dyb, 1, False)),
             quant_both_bytes(M, N))):
        dt = timed(fn)
        per_op[name] = {"oracle_GB/s": round(nbytes / dt / 1e9, 3), "oracle_s": round(dt, 3),
                        "sample": "the full tensor"}
    del xb, wb, dyb

    # GEMMs: codes and scales with the workload's value ranges (the oracle's cost does not depend on them)
    rng = np.random.default_rng(99)
    a_mk = rng.integers(0, 0x7E, (M, K), dtype=np.uint8)
    b_nk = rng.integers(0, 0x7E, (N, K), dtype=np.uint8)
    s_km = rng.uniform(1e-3, 1e-2, (K // 128, M)).astype(np.float32)
    s_blk = rng.uniform(1e-5, 1e-4, (N // 128, K // 128)).astype(np.float32)
    a_mn = rng.integers(0, 0x7E, (M, N), dtype=np.uint8)
    s_nm = rng.uniform(1e-3, 1e-2, (N // 128, M)).astype(np.float32)
    at_nm = rng.integers(0, 0x7E, (N, M), dtype=np.uint8)
    at_km = rng.integers(0, 0x7E, (K, M), dtype=np.uint8)
    s_mn = rng.uniform(1e-3, 1e-2, (M // 128, N)).astype(np.float32)
    s_mk = rng.uniform(1e-3, 1e-2, (M // 128, K)).astype(np.float32)
    gemms = (("fprop", M * N, K, lambda p: oracle.gemm_fprop(a_mk, s_km, b_nk, s_blk, out_bf16=True, pts=p,
                                                               want_exact=False)),
             ("dgrad", M * K, N, lambda p: oracle.gemm_dgrad(a_mn, s_nm, b_nk, s_blk, pts=p, want_exact=False)),
             ("wgrad", N * K, M, lambda p: oracle.gemm_wgrad(at_nm, s_mn, at_km, s_mk, pts=p, want_exact=False)))
    left = max(budget_s - (time.perf_counter() - t_start), 6.0)
    total_flop, total_s = 0.0, 0.0
    for name, n_out, depth, fn in gemms:
        npts, flop, el = 256, 0.0, 0.0
        while el < left / 3 and npts <= 1 << 22:
            pts = rng.integers(0, n_out, npts, dtype=np.int64)
            el += timed(lambda: fn(pts))
            flop += 2.0 * depth * npts
            npts *= 2
        per_op[name] = {"oracle_TFLOP/s": round(flop / el / 1e12, 6), "oracle_s": round(el, 2),
                        "sample": f"{int(flop / (2 * depth))} sampled outputs, each a {depth}-deep promoted dot product"}
        total_flop += flop
        total_s += el
    if gpu_kernels:
        for name, entry in per_op.items():
            g = gpu_kernels.get(name)
            if not g:
                continue
            if "TFLOP/s" in g:
                entry["gpu_TFLOP/s"] = g["TFLOP/s"]
                entry["gpu_over_oracle"] = round(g["TFLOP/s"] / entry["oracle_TFLOP/s"], 1)
            elif "GB/s" in g:
                entry["gpu_GB/s"] = g["GB/s"]
                entry["gpu_over_oracle"] = round(g["GB/s"] / entry["oracle_GB/s"], 1)
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    return {"value": total_flop / total_s / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "cpu_model": model,
            "kind": "oracle",
            "sample": f"sampled outputs of the step's three 4096x18432x7168 GEMMs ({total_s:.1f} s), plus the "
                      f"step's quantizers on their full tensors (per_op)",
            "per_op": per_op}


if __name__ == "__main__":
    main()
