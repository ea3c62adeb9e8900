#!/usr/bin/env python3
"""Benchmark of the fp32 matrix product and implicit-GEMM convolution on one MI355X.

A step is one fast-mode 4096^3 matrix product (N(0,1) inputs with 0.1% special
values at seeded positions) through the C ABI, inputs resident in HBM.  After
W untimed steps, K steps are timed back to back between HIP events on the
stream the kernels run on; the JSON line reports GFLOP/s, the roofline
fraction of the dominant kernel, and the CPU oracle timed on a bounded
sample.  The other workloads (exact mode at 4096^3, 256^3, the ragged,
prefill and skinny products, the ResNet-50 convolution chain at batch 1 and
8, the grouped/dilated and 1-D convolutions) are timed in both modes under
"extra": 2 warm-up calls, calls repeated for at least 80 ms between events,
the median of 3 such repetitions.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fp32 GFLOP/s (exact & fast) at 4096^3 + ResNet-50 conv chain ms; % fp32 peak"
PEAK_FP32_TFLOPS = 157.3        # MI355X dense fp32 (matrix and packed vector)
# Exact mode: the matrix cores form each rounded product and a separately
# rounded non-packed VALU add (32 lanes per clock per SIMD) takes each term;
# on one SIMD the two do not overlap (measured), so a term costs 1/32 + 1/32
# clock per SIMD: half the fp32 peak.
EXACT_CEILING_TFLOPS = 78.65
HBM_GBPS = 8000.0
COLD_BYTES = 600 << 20  # rotated input copies beyond the 256 MB last-level cache and the L2s
# HBM bytes per launch of the headline kernel, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE runs scaled by a 1 GiB copy (the summary under profiles/ gives
# the commands and counts).  Valid only for the kernel build it was measured
# on (None until the counters are taken again after a change to it):
# FETCH_SIZE 196 767.1 KiB x 2.00 + WRITE_SIZE 65 536.0 KiB x 1.00.
HEADLINE_TRAFFIC = {"variant": 17, "kernel": "og::mfma_kernel<1, 256, 256, 4, 2, 0, true, true, 2, 32>",
                    "bytes": 470087885}
PAGES_RESNET_CPU_MS = {"16 threads": 12.3, "32 threads": 11.1}  # 16-core Zen 4, fast mode


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", default=None,
                    help="time one workload only (for profiling): gemm4096_fast, gemm4096_exact, "
                         "resnet_b1, resnet_b8, epilogue, skinny, prefill, grouped, conv1d, conv1x1, ragged, "
                         "gemm256, dw_b1, dw_b8, se, single_column, nt_prefill, nt_single_row, nt_rows8, model_rows, "
                         "copy (a 1 GiB device copy, to scale the HBM byte counters), "
                         "layer (one ResNet-50 layer: --layer, --batch, --variant, --mode; "
                         "--warmup then --steps calls)")
    ap.add_argument("--layer", default="layer3.1.c2",
                    help="with --only layer: the ResNet-50 layer to time (e.g. layer3.1.c2)")
    ap.add_argument("--batch", type=int, default=8, help="with --only layer: the batch")
    ap.add_argument("--variant", type=int, default=0,
                    help="with --only layer: the kernel variant forced (0: the automatic choice)")
    ap.add_argument("--mode", default="fast", help="with --only layer: exact, fast or fast_mfma")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--extra-out", default=os.path.join("gpurun_out", "bench_extra.json"),
                    help="file for the other workloads' numbers (relative to the repository)")
    return ap.parse_args()


class Timer:
    """HIP events on the current torch stream (the stream libog launches on)."""

    def __init__(self, torch):
        self.torch = torch

    def time_calls(self, fn, calls: int) -> float:
        t = self.torch
        s = t.cuda.current_stream()
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        e0.record(s)
        for _ in range(calls):
            fn()
        e1.record(s)
        t.cuda.synchronize()
        return e0.elapsed_time(e1) / calls  # ms per call

    def graph(self, fn, calls: int = 1):
        """`calls` calls of fn captured in one HIP graph (fn launches kernels only)."""
        t = self.torch
        fn()
        t.cuda.synchronize()
        s = t.cuda.Stream()
        s.wait_stream(t.cuda.current_stream())
        g = t.cuda.CUDAGraph()
        with t.cuda.stream(s):
            with t.cuda.graph(g, stream=s):
                for _ in range(calls):
                    fn()
        t.cuda.synchronize()
        return g

    def spike(self, fn, min_ms: float = 80.0, reps: int = 3) -> float:
        """2 warm-ups; calls repeated for >= min_ms; median of `reps` means (ms per call)."""
        fn()
        fn()
        one = self.time_calls(fn, 1)
        calls = max(1, int(min_ms / max(one, 1e-3)) + 1)
        return statistics.median(self.time_calls(fn, calls) for _ in range(reps))


def dev_strided(torch, case_A, ld):
    rows, cols = case_A.shape
    buf = torch.empty((rows, ld), dtype=torch.float32, device="cuda")
    buf[:, :cols] = torch.from_numpy(case_A).cuda()
    return buf[:, :cols]


def gemm_workload(torch, og, case):
    A = dev_strided(torch, case.A, case.lda)
    B = dev_strided(torch, case.B, case.ldb)
    C = torch.empty((case.m, case.ldc), dtype=torch.float32, device="cuda")[:, :case.n]
    return A, B, C


def conv_chain(torch, og, synth, batch):
    layers = []
    for i, s in enumerate(synth.resnet50_convs(batch)):
        x, w = synth.conv_inputs(s, synth.seed_for(4, i + (0 if batch == 1 else 100)))
        dx, dw = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
        y = og.conv2d(dx, dw, stride=s.stride, pad=s.pad, dil=s.dil, groups=s.groups)
        layers.append((s, dx, dw, y))
    return layers


def conv_macs(og, s):
    oh = og.conv2d_out_size(s.H, s.KH, s.stride[0], s.pad[0], s.pad[2], s.dil[0])
    ow = og.conv2d_out_size(s.W, s.KW, s.stride[1], s.pad[1], s.pad[3], s.dil[1])
    return s.N * s.Cout * oh * ow * (s.Cin // s.groups) * s.KH * s.KW


def chain_entry_impl(torch, og, synth, timer, shapes, config, seed0):
    """A list of convolutions timed as one chain (HIP graph and eager launches)
    and one by one, with their algorithmic bytes (x, w and y once each)."""
    layers = []
    for i, s in enumerate(shapes):
        x, w = synth.conv_inputs(s, synth.seed_for(config, seed0 + i))
        dx, dw = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
        y = og.conv2d(dx, dw, stride=s.stride, pad=s.pad, dil=s.dil, groups=s.groups)
        layers.append((s, dx, dw, y))
    macs = sum(conv_macs(og, s) for s, *_ in layers)
    nbytes = sum(4.0 * (dx.numel() + dw.numel() + y.numel()) for _, dx, dw, y in layers)
    ent = {"layers": len(layers), "gflop": round(2 * macs / 1e9, 4),
           "mbytes": round(nbytes / 1e6, 3)}
    for mode in ("fast", "exact"):
        g = timer.graph(lambda: run_chain(og, layers, mode))
        ms = timer.spike(g.replay)
        ms_eager = timer.spike(lambda: run_chain(og, layers, mode))
        ent[mode] = {"us": round(ms * 1e3, 2), "us_eager_launches": round(ms_eager * 1e3, 2),
                     "gflops": round(2 * macs / (ms * 1e-3) / 1e9, 1),
                     "tensor_gbps": round(nbytes / (ms * 1e-3) / 1e9, 1)}
        del g
    per = {}
    for s, dx, dw, y in layers:
        e = {"shape": repr(s), "mbytes": round(4.0 * (dx.numel() + dw.numel() + y.numel()) / 1e6, 3)}
        for mode in ("fast", "exact"):
            call = (lambda s_, dx_, dw_, y_, m_: lambda: og.conv2d(
                dx_, dw_, stride=s_.stride, pad=s_.pad, dil=s_.dil, groups=s_.groups, mode=m_,
                out=y_))(s, dx, dw, y, mode)
            g = timer.graph(lambda: [call() for _ in range(20)])
            us = timer.spike(g.replay, min_ms=30.0) / 20 * 1e3
            e[f"{mode}_us"] = round(us, 2)
            e[f"{mode}_gbps"] = round(e["mbytes"] * 1e6 / (us * 1e-6) / 1e9, 1)
            del g
        per[s.name] = e
    ent["per_layer"] = per
    del layers
    return ent


def model_rows(torch, og, synth, timer):
    """Per model: each distinct shape timed alone (20 calls replayed from a HIP
    graph, 2 warm-ups, >= 20 ms, median of 3), summed as count x time, both
    modes, and the exact / fast ratio.  Linear layers run as products with
    N x K weights (og_gemm_nt_f32), A N(0,1), weights N(0, 0.02)."""
    def timed(call):
        g = timer.graph(lambda: [call() for _ in range(20)])
        us = timer.spike(g.replay, min_ms=20.0) / 20 * 1e3
        del g
        return us

    def conv_shapes(shapes):
        groups = {}
        for s in shapes:
            key = (s.N, s.Cin, s.H, s.W, s.Cout, s.KH, s.KW, s.stride, s.pad, s.dil, s.groups)
            groups.setdefault(key, [s, 0])[1] += 1
        return list(groups.values())

    rows = {}
    models = {"bert_base_32x128": ("bert_base_4096", []), "bert_base_128": ("bert_base_128", []),
              "minilm_l6_32x128": ("minilm_l6_4096", []),
              "whisper_small_encoder_1500": ("whisper_small_enc_1500", synth.whisper_small_frontend()),
              "resnet50_b1": (None, synth.resnet50_convs(1)),
              "mobilenetv3_large_b1": (None, synth.mobilenetv3_large_convs(1))}
    for name, (lin, convs) in models.items():
        ent = {"shapes": 0, "gflop": 0.0, "fast_us": 0.0, "exact_us": 0.0}
        for i, (lname, m, n, k, count) in enumerate(synth.transformer_linear_shapes(lin) if lin else []):
            A = torch.from_numpy(synth.normal((m, k), synth.seed_for(8, 10 * i))).cuda()
            W = torch.from_numpy(synth.normal((n, k), synth.seed_for(8, 10 * i + 1), 0.02)).cuda()
            C = torch.empty((m, n), dtype=torch.float32, device="cuda")
            ent["shapes"] += 1
            ent["gflop"] += count * 2.0 * m * n * k / 1e9
            for mode in ("fast", "exact"):
                ent[f"{mode}_us"] += count * timed(lambda: og.gemm_nt(A, W, mode, out=C))
            del A, W, C
        for i, (s, count) in enumerate(conv_shapes(convs)):
            x, w = synth.conv_inputs(s, synth.seed_for(8, 500 + i))
            dx, dw = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
            y = og.conv2d(dx, dw, stride=s.stride, pad=s.pad, dil=s.dil, groups=s.groups)
            ent["shapes"] += 1
            ent["gflop"] += count * 2.0 * conv_macs(og, s) / 1e9
            for mode in ("fast", "exact"):
                ent[f"{mode}_us"] += count * timed(lambda: og.conv2d(
                    dx, dw, stride=s.stride, pad=s.pad, dil=s.dil, groups=s.groups, mode=mode, out=y))
            del dx, dw, y
        ent["gflop"] = round(ent["gflop"], 3)
        for mode in ("fast", "exact"):
            ent[f"{mode}_us"] = round(ent[f"{mode}_us"], 1)
            ent[f"{mode}_tflops"] = round(ent["gflop"] * 1e3 / ent[f"{mode}_us"], 2)
        ent["exact_over_fast"] = round(ent["exact_us"] / ent["fast_us"], 3)
        rows[name] = ent
    return rows


def run_chain(og, layers, mode):
    for s, dx, dw, y in layers:
        og.conv2d(dx, dw, stride=s.stride, pad=s.pad, dil=s.dil, groups=s.groups, mode=mode,
                  out=y)


def extras(torch, og, synth, timer, only=None):
    out = {}

    def want(name):
        return only is None or only == name

    def graph_ms(calls):
        """ms per call of `calls` (a list of closures) replayed from one HIP graph."""
        g = timer.graph(lambda: [c() for c in calls])
        ms = timer.spike(g.replay) / len(calls)
        del g
        return ms

    def gemm_entry(case, modes=("fast", "exact", "fast_mfma"), bytes_moved=None, cold_copies=0):
        A, B, C = gemm_workload(torch, og, case)
        # cold: each call reads its own copy of B, the copies together larger
        # than the last-level cache, so B comes from HBM
        Bs = [dev_strided(torch, case.B, case.ldb) for _ in range(cold_copies)]
        ent = {"m": case.m, "n": case.n, "k": case.k, "lda": case.lda, "ldb": case.ldb,
               "ldc": case.ldc}
        for mode in modes:
            # kernel time: calls replayed from a HIP graph (no host time
            # between launches); also the calls issued one by one from Python
            ms = graph_ms([lambda: og.gemm(A, B, mode, out=C)] * 20)
            ms_eager = timer.spike(lambda: og.gemm(A, B, mode, out=C))
            ent[mode] = {"us": round(ms * 1e3, 2), "us_eager_launches": round(ms_eager * 1e3, 2),
                         "gflops": round(case.flops / (ms * 1e-3) / 1e9, 1),
                         "frac_peak": round(case.flops / (ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 4)}
            if mode == "exact":
                ent[mode]["frac_exact_ceiling"] = round(
                    case.flops / (ms * 1e-3) / 1e12 / EXACT_CEILING_TFLOPS, 4)
            if bytes_moved:
                ent[mode]["hbm_gbps_hot"] = round(bytes_moved / (ms * 1e-3) / 1e9, 1)
            if Bs:
                ms_cold = graph_ms([(lambda b: lambda: og.gemm(A, b, mode, out=C))(b) for b in Bs])
                ent[mode]["us_cold"] = round(ms_cold * 1e3, 2)
                ent[mode]["hbm_gbps_cold"] = round(bytes_moved / (ms_cold * 1e-3) / 1e9, 1)
        del A, B, C, Bs
        return ent

    def conv_entry(s, dist, seed, cold_bytes=0):
        x, w = synth.conv_inputs(s, seed, dist)
        dx, dw = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
        y = og.conv2d(dx, dw, stride=s.stride, pad=s.pad, dil=s.dil, groups=s.groups)
        macs = conv_macs(og, s)
        nbytes = 4.0 * (x.size + w.size + y.numel())
        xs = [dx.clone() for _ in range(-(-cold_bytes // (4 * x.size)))] if cold_bytes else []
        ent = {"shape": repr(s), "gflop": round(2 * macs / 1e9, 4)}
        for mode in ("fast", "exact", "fast_mfma"):
            call = lambda xx: og.conv2d(xx, dw, stride=s.stride, pad=s.pad, dil=s.dil,
                                        groups=s.groups, mode=mode, out=y)
            ms = graph_ms([lambda: call(dx)] * 20)
            ms_eager = timer.spike(lambda: call(dx))
            ent[mode] = {"us": round(ms * 1e3, 2), "us_eager_launches": round(ms_eager * 1e3, 2),
                         "gflops": round(2 * macs / (ms * 1e-3) / 1e9, 1),
                         "tensor_gbps_hot": round(nbytes / (ms * 1e-3) / 1e9, 1)}
            if xs:
                ms_cold = graph_ms([(lambda xx: lambda: call(xx))(xx) for xx in xs])
                ent[mode]["us_cold"] = round(ms_cold * 1e3, 2)
                ent[mode]["tensor_gbps_cold"] = round(nbytes / (ms_cold * 1e-3) / 1e9, 1)
        del dx, dw, y, xs
        return ent

    def chain_entry(shapes, config, seed0):
        return chain_entry_impl(torch, og, synth, timer, shapes, config, seed0)

    if only == "copy":
        x = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        x.fill_(1.0)
        ms = timer.spike(lambda: y.copy_(x))
        out["copy_1GiB"] = {"bytes_read": x.numel() * 4, "bytes_written": y.numel() * 4,
                            "us": round(ms * 1e3, 1),
                            "gbps": round(2 * x.numel() * 4 / (ms * 1e-3) / 1e9, 1)}
        return out
    if want("gemm4096_exact") and only is not None:
        out["gemm_4096"] = gemm_entry(synth.gemm_4096(), modes=("exact",))
        return out
    if want("gemm256"):
        log("extra: gemm 256^3")
        out["gemm_256"] = gemm_entry(synth.gemm_square256())
    if want("ragged"):
        log("extra: ragged")
        out["gemm_1000x777x1531_ld13"] = gemm_entry(synth.gemm_ragged())
    if want("prefill"):
        log("extra: prefill")
        out["gemm_prefill_512x11008x4096"] = gemm_entry(synth.gemm_prefill())
    if want("skinny"):
        log("extra: skinny")
        c = synth.gemm_skinny()
        out["gemm_skinny_1x4096x4096"] = gemm_entry(c, bytes_moved=4.0 * (c.k * c.n + c.k + c.n),
                                                    cold_copies=10)
    for batch in (1, 8):
        name = f"resnet_b{batch}"
        if not want(name):
            continue
        log(f"extra: resnet50 chain batch {batch}")
        layers = conv_chain(torch, og, synth, batch)
        macs = sum(conv_macs(og, s) for s, *_ in layers)
        ent = {"layers": len(layers), "gflop": round(2 * macs / 1e9, 3)}
        for mode in ("fast", "exact", "fast_mfma"):
            # the 53 launches replayed from one HIP graph (no host time between
            # kernels), and issued one by one from Python
            g = timer.graph(lambda: run_chain(og, layers, mode))
            ms = timer.spike(g.replay)
            ms_eager = timer.spike(lambda: run_chain(og, layers, mode))
            ent[mode] = {"ms": round(ms, 4), "ms_eager_launches": round(ms_eager, 4),
                         "gflops": round(2 * macs / (ms * 1e-3) / 1e9, 1),
                         "frac_peak": round(2 * macs / (ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 4)}
            del g
        # per distinct shape: 20 calls of the layer replayed from a HIP graph;
        # count x time summed over the shapes should agree with the chain
        shapes = {}
        for s, dx, dw, y in layers:
            key = (s.Cin, s.H, s.Cout, s.KH, s.stride)
            if key in shapes:
                shapes[key][1] += 1
            else:
                shapes[key] = [(s, dx, dw, y), 1]
        per = {}
        for (s, dx, dw, y), cnt in shapes.values():
            e = {"count": cnt, "shape": f"{s.Cin}->{s.Cout} {s.H}x{s.W} k{s.KH}x{s.KW} s{s.stride[0]}"}
            for mode in ("fast", "exact", "fast_mfma"):
                call = (lambda s_, dx_, dw_, y_, m_: lambda: og.conv2d(
                    dx_, dw_, stride=s_.stride, pad=s_.pad, dil=s_.dil, groups=s_.groups, mode=m_,
                    out=y_))(s, dx, dw, y, mode)
                g = timer.graph(lambda: [call() for _ in range(20)])
                e[f"{mode}_us"] = round(timer.spike(g.replay, min_ms=30.0) / 20 * 1e3, 2)
                del g
            per[s.name] = e
        ent["per_shape"] = per
        for mode in ("fast", "exact", "fast_mfma"):
            ent[mode]["sum_count_x_shape_ms"] = round(
                sum(e["count"] * e[f"{mode}_us"] for e in per.values()) / 1e3, 4)
        if batch == 1:
            ent["pages_cpu_context_ms"] = PAGES_RESNET_CPU_MS
        out[f"resnet50_chain_b{batch}"] = ent
        del layers
    if want("epilogue"):
        # the batch-8 chain with each convolution's bias, ReLU and residual:
        # fused into the convolution's stores, against the same three steps
        # as separate elementwise passes over the output
        log("extra: fused epilogue on the resnet50 batch-8 chain")
        layers = conv_chain(torch, og, synth, 8)
        epi = []
        for i, (s, dx, dw, y) in enumerate(layers):
            b = torch.from_numpy(synth.normal((s.Cout,), synth.seed_for(4, 300 + i), 0.1)).cuda()
            r = torch.from_numpy(synth.normal(tuple(y.shape), synth.seed_for(4, 400 + i))).cuda()
            epi.append((b, r))
        out_bytes = sum(4.0 * y.numel() for *_, y in layers)
        ent = {"layers": len(layers), "epilogue": "y = relu(conv + bias) + residual",
               "output_mb": round(out_bytes / 1e6, 1)}

        def fused(mode):
            for (s, dx, dw, y), (b, r) in zip(layers, epi):
                og.conv2d(dx, dw, stride=s.stride, pad=s.pad, dil=s.dil, groups=s.groups,
                          mode=mode, out=y, bias=b, act="relu", residual=r)

        def separate(mode):
            run_chain(og, layers, mode)
            for (s, dx, dw, y), (b, r) in zip(layers, epi):
                y.add_(b.view(1, -1, 1, 1)).relu_().add_(r)

        for mode in ("fast", "exact"):
            row = {}
            for key, fn in (("conv_only_ms", lambda: run_chain(og, layers, mode)),
                            ("fused_ms", lambda: fused(mode)),
                            ("separate_passes_ms", lambda: separate(mode))):
                g = timer.graph(fn)
                row[key] = round(timer.spike(g.replay), 4)
                del g
            ent[mode] = row
        out["resnet50_b8_epilogue"] = ent
        del layers, epi
    for name, shape_fn, dist in (("grouped", synth.grouped_dilated, "uniform"),
                                 ("conv1d", synth.conv1d_h1, "uniform")):
        if not want(name):
            continue
        log(f"extra: {name}")
        s = shape_fn()
        out[s.name] = conv_entry(s, dist, synth.seed_for(5, 0),
                                 cold_bytes=COLD_BYTES if name == "grouped" else 0)
    for batch in (1, 8):
        name = f"dw_b{batch}"
        if want(name):
            log(f"extra: MobileNetV3-large depthwise convolutions, batch {batch}")
            out[f"mobilenetv3_depthwise_b{batch}"] = chain_entry(
                synth.mobilenetv3_large_depthwise(batch), 6, 100 * batch)
    if want("se"):
        log("extra: MobileNetV3-large squeeze-and-excitation convolutions, batch 1")
        out["mobilenetv3_se_b1"] = chain_entry(synth.mobilenetv3_large_se(1), 7, 0)
    if want("single_column"):
        log("extra: single-column product")
        c = synth.gemm_single_column()
        out["gemm_single_column_4096x1x4096"] = gemm_entry(
            c, bytes_moved=4.0 * (c.m * c.k + c.k + c.m))
    for name, m in (("nt_prefill", 512), ("nt_single_row", 1), ("nt_rows8", 8)):
        if not want(name):
            continue
        log(f"extra: {name}")
        n = 11008 if m == 512 else 4096
        A = torch.from_numpy(synth.normal((m, 4096), synth.seed_for(3, 20))).cuda()
        Bt = torch.from_numpy(synth.normal((n, 4096), synth.seed_for(3, 21), 0.02)).cuda()
        C = torch.empty((m, n), dtype=torch.float32, device="cuda")
        flops, nbytes = 2.0 * m * n * 4096, 4.0 * (m * 4096 + n * 4096 + m * n)
        ent = {"m": m, "n": n, "k": 4096, "layout": "B given as n x k (weights N x K)"}
        for mode in ("fast", "exact", "fast_mfma"):
            ms = graph_ms([lambda: og.gemm_nt(A, Bt, mode, out=C)] * 20)
            ent[mode] = {"us": round(ms * 1e3, 2), "gflops": round(flops / (ms * 1e-3) / 1e9, 1),
                         "frac_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 4),
                         "hbm_gbps_hot": round(nbytes / (ms * 1e-3) / 1e9, 1)}
        out[f"gemm_nt_{m}x{n}x4096"] = ent
        del A, Bt, C
    if want("model_rows"):
        # the pages' model rows: over the distinct matrix-product and
        # convolution shapes of one model, count x time summed, exact / fast
        log("extra: model rows")
        out["model_rows"] = model_rows(torch, og, synth, timer)
    if want("conv1x1"):
        # the 1x1 layers of the batch-8 chain, hot and cold (HBM-bound shapes)
        log("extra: 1x1 layers of the batch-8 chain")
        seen, ent = set(), {}
        for i, s in enumerate(synth.resnet50_convs(8)):
            key = (s.Cin, s.H, s.Cout, s.stride)
            if s.KH != 1 or key in seen:
                continue
            seen.add(key)
            ent[s.name] = conv_entry(s, "normal", synth.seed_for(4, 200 + i), cold_bytes=COLD_BYTES)
        out["resnet50_b8_1x1_layers"] = ent
    return out


def cpu_oracle_table(synth, seconds_each=2.0):
    """The oracle at all threads and at 1 thread, exact and fast, each on the
    first rows of the 4096^3 product (whole calls for >= seconds_each)."""
    import oracle
    orc = oracle.get()
    c = synth.gemm_4096()
    full = orc.num_threads()
    out = {"cpu_model": cpu_model(), "logical_cpus": os.cpu_count(),
           "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS"), "runs": []}
    try:
        for threads in (full, 1):
            orc.set_num_threads(threads)
            for mode, name in ((1, "fast"), (0, "exact")):
                rows = 16 if threads > 1 else 2
                orc.gemm(c.A[:rows], c.B, mode, rowwise=True)  # warm-up
                calls, t0 = 0, time.perf_counter()
                while True:
                    orc.gemm(c.A[:rows], c.B, mode, rowwise=True)
                    calls += 1
                    dt = time.perf_counter() - t0
                    if dt >= seconds_each:
                        break
                out["runs"].append({"threads": threads, "mode": name, "rows": rows, "calls": calls,
                                    "gflops": round(2.0 * calls * rows * c.n * c.k / dt / 1e9, 3)})
    finally:
        orc.set_num_threads(full)
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(synth, seconds):
    """The oracle (fast mode, its row-wise loop) on a bounded sample of the 4096^3 rows."""
    import oracle
    orc = oracle.get()
    c = synth.gemm_4096()
    rows = 8
    t0 = time.perf_counter()
    orc.gemm(c.A[:rows], c.B, 1, rowwise=True)
    dt = time.perf_counter() - t0
    rows = int(min(c.m, max(rows, rows * seconds / max(dt, 1e-6))))
    calls = 0
    t0 = time.perf_counter()
    while True:  # whole calls until the sample has run for `seconds`
        orc.gemm(c.A[:rows], c.B, 1, rowwise=True)
        calls += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    flops = 2.0 * calls * rows * c.n * c.k
    return {"value": round(flops / dt / 1e9, 3), "unit": "GFLOP/s", "cores": orc.num_threads(),
            "kind": "oracle",
            "sample": f"fast mode, rows 0..{rows - 1} of the 4096^3 product (all 4096 columns, "
                      f"k = 4096), {calls} call(s) of the oracle's row-wise loop, {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for "
              f"--gpus {args.gpus}); the matrix product and convolution shard without any "
              "exchange, by rows/columns of C or by image/group, each GPU running the one-GPU "
              "kernel on its share.", file=sys.stderr)
        sys.exit(2)
    import torch

    import fp32_blocked_gemm_amd as og
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    og.lib()
    timer = Timer(torch)

    if args.only == "layer":
        # one layer, its calls issued back to back (for profiling a kernel)
        s = [c for c in synth.resnet50_convs(args.batch) if c.name == args.layer]
        if not s:
            print(f"no ResNet-50 layer {args.layer}", file=sys.stderr)
            sys.exit(2)
        s = s[0]
        x, w = synth.conv_inputs(s, 1)
        dx, dw = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
        og.set_variant(args.variant)
        call = lambda: og.conv2d(dx, dw, stride=s.stride, pad=s.pad, dil=s.dil, groups=s.groups,
                                 mode=args.mode)
        y = call()
        for _ in range(args.warmup):
            og.conv2d(dx, dw, stride=s.stride, pad=s.pad, dil=s.dil, groups=s.groups,
                      mode=args.mode, out=y)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            og.conv2d(dx, dw, stride=s.stride, pad=s.pad, dil=s.dil, groups=s.groups,
                      mode=args.mode, out=y)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / max(args.steps, 1) * 1e3
        print(json.dumps({"only": "layer", "layer": args.layer, "batch": args.batch,
                          "variant": args.variant, "mode": args.mode, "shape": repr(s),
                          "us_per_call": round(us, 2),
                          "gflops": round(2 * conv_macs(og, s) / (us * 1e-6) / 1e9, 1)}), flush=True)
        return
    if args.only not in (None, "gemm4096_fast"):
        log(f"only: {args.only}")
        res = extras(torch, og, synth, timer, only=args.only)
        print(json.dumps({"only": args.only, "extra": res}), flush=True)
        return

    # The headline's inputs are made first and the other workloads run before
    # it, so its W warm-up and K timed steps follow a minute of GPU work with
    # no idle gap: the first ~30 launches after an idle GPU run up to 15 %
    # slower while its clock ramps up (measured), which a 20-step region
    # would mostly time.
    case = synth.gemm_4096()
    A, B, C = gemm_workload(torch, og, case)
    extra = {}
    if args.only is None and not args.no_extra:
        extra["gemm_4096_exact"] = extras(torch, og, synth, timer,
                                          only="gemm4096_exact")["gemm_4096"]["exact"]
        extra.update(extras(torch, og, synth, timer))
    log("headline: fast-mode 4096^3 matrix product")
    for _ in range(args.warmup):
        og.gemm(A, B, "fast", out=C)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ms = timer.time_calls(lambda: og.gemm(A, B, "fast", out=C), args.steps)
    wall = time.perf_counter() - wall0
    flops = case.flops
    value = flops / (ms * 1e-3) / 1e9
    achieved = flops / (ms * 1e-3) / 1e12
    # the variant the library's automatic choice ran (og_gemm_choice)
    variant = og.gemm_choice(4096, 4096, 4096, "fast")
    same_kernel = variant == HEADLINE_TRAFFIC["variant"]
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "fp32 GEMM m=n=k=4096, fast mode (ordered FMA), row-major, "
                               "N(0,1) with 0.1% special values", "m": 4096, "n": 4096, "k": 4096,
                   "mode": "fast", "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_TFLOPS, 4),
                     # the counters hold for the kernel they were taken on:
                     # none when the library's choice for 4096^3 is another
                     "traffic": (None if HEADLINE_TRAFFIC["bytes"] is None or not same_kernel
                                 else round(HEADLINE_TRAFFIC["bytes"])),
                     "traffic_unit": "bytes per launch (HBM, counter-measured)",
                     "variant": variant,
                     "kernel": HEADLINE_TRAFFIC["kernel"] if same_kernel else f"variant {variant}",
                     "wall_s_timed_region": round(wall, 3)},
    }
    del A, B, C
    if extra:
        line["summary"] = summarize(extra)
    if args.only is None and not args.no_cpu:
        log("cpu baseline: oracle on a bounded sample")
        line["cpu_baseline"] = cpu_baseline(synth, args.cpu_seconds)
        extra["cpu_oracle"] = cpu_oracle_table(synth)
    if extra:
        # every workload's numbers: to a file and, as one line, to stderr; the
        # last line of stdout stays the short record
        out = os.path.join(ROOT, args.extra_out) if not os.path.isabs(args.extra_out) else args.extra_out
        try:
            os.makedirs(os.path.dirname(out), exist_ok=True)
            with open(out, "w") as f:
                json.dump(extra, f, indent=1)
            line["extra_file"] = os.path.relpath(out, ROOT)
        except OSError as e:
            log(f"could not write {out}: {e}")
        print("extra: " + json.dumps(extra), file=sys.stderr, flush=True)
    print(json.dumps(line), flush=True)


def summarize(ex):
    """A few figures of the other workloads for the short record (the full
    set goes to the extra file)."""
    def get(*keys):
        d = ex
        for k in keys:
            if not isinstance(d, dict) or k not in d:
                return None
            d = d[k]
        return d

    out = {"gemm_4096_exact": {"ms": None if get("gemm_4096_exact", "us") is None
                               else round(get("gemm_4096_exact", "us") / 1e3, 4),
                               "tflops": None if get("gemm_4096_exact", "gflops") is None
                               else round(get("gemm_4096_exact", "gflops") / 1e3, 2),
                               "frac_exact_ceiling": get("gemm_4096_exact", "frac_exact_ceiling")}}
    for b in (1, 8):
        out[f"resnet50_chain_b{b}_ms"] = {m: get(f"resnet50_chain_b{b}", m, "ms")
                                          for m in ("fast", "exact", "fast_mfma")
                                          if get(f"resnet50_chain_b{b}", m, "ms") is not None}
    for key, name in (("gemm_256", "gemm_256_us"), ("gemm_1000x777x1531_ld13", "ragged_us"),
                      ("gemm_prefill_512x11008x4096", "prefill_us"),
                      ("gemm_skinny_1x4096x4096", "skinny_us"),
                      ("grouped_g32_d2_s2", "grouped_dilated_us"), ("conv1d_w4096_k5", "conv1d_us")):
        out[name] = {m: get(key, m, "us") for m in ("fast", "exact", "fast_mfma")
                     if get(key, m, "us") is not None}
    return out


if __name__ == "__main__":
    main()
