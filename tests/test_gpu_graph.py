"""Launches captured in a HIP graph give the same bits on every replay as
the same calls issued one by one (the benchmark replays the convolution
chain from a graph).  Replays are interleaved with eager launches that
overwrite the outputs, and every replay is checked."""
import numpy as np
import pytest

import fp32_blocked_gemm_amd as og
import synth
from gpu_util import assert_same_bits, say, to_host, torch

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    t = torch()
    shapes = [s for s in synth.resnet50_convs(1)
              if s.name in ("stem", "layer1.0.c2", "layer2.0.down", "layer3.1.c1", "layer4.1.c2")]
    layers = []
    for i, s in enumerate(shapes):
        x, w = synth.conv_inputs(s, synth.seed_for(6, i))
        dx, dw = t.from_numpy(x).cuda(), t.from_numpy(w).cuda()
        layers.append((s, dx, dw, og.conv2d(dx, dw, stride=s.stride, pad=s.pad, dil=s.dil)))
    rng = np.random.default_rng(6)
    A = t.from_numpy(rng.standard_normal((300, 517)).astype(np.float32)).cuda()
    B = t.from_numpy(rng.standard_normal((517, 70)).astype(np.float32)).cuda()
    C = t.empty((300, 70), device="cuda")

    def run(mode):
        for s, dx, dw, y in layers:
            og.conv2d(dx, dw, stride=s.stride, pad=s.pad, dil=s.dil, mode=mode, out=y)
        og.gemm(A, B, mode, out=C)

    for mode in ("exact", "fast"):
        run(mode)
        t.cuda.synchronize()
        want = [to_host(y).copy() for *_, y in layers] + [to_host(C).copy()]
        side = t.cuda.Stream()
        side.wait_stream(t.cuda.current_stream())
        g = t.cuda.CUDAGraph()
        with t.cuda.stream(side):
            with t.cuda.graph(g, stream=side):
                run(mode)
        t.cuda.synchronize()
        for rep in range(4):
            for *_, y in layers:
                y.fill_(float("nan"))
            C.fill_(float("nan"))
            run("fast" if mode == "exact" else "exact")  # eager work between replays
            t.cuda.synchronize()
            g.replay()
            t.cuda.synchronize()
            say(f"graph replay {rep} mode {mode}")
            got = [to_host(y) for *_, y in layers] + [to_host(C)]
            for gg, ww, name in zip(got, want, [s.name for s, *_ in layers] + ["gemm"]):
                assert_same_bits(gg, ww, f"replay {rep} {name} mode {mode}")
