"""Measures the regret of libog's automatic kernel choice (fast or exact mode): for
each shape of a set, the time of the automatic choice (variant 0) over the
best time of every variant that runs the shape, each forced with
og_set_variant.  Needs a GPU.

Two sets of shapes.  "fit": the shapes the fast-mode launch-time table was
fitted to -- ResNet-50's convolutions at batch 1, 2, 3, 4, 5, 6, 8, 12 and
16, MobileNetV3-large's ungrouped convolutions at batch 1, 2, 4, 6 and 8,
twelve 3x3 convolutions of other widths and 72 seeded random matrix
products.  "heldout": shapes the fit did not see -- ResNet-50 at batch 7
and 10, MobileNetV3-large at batch 3 and 5, four more 3x3 convolutions and
24 random products of another seed.  "large" (fitted too) and
"large_heldout": products of the sizes of a language model's layers, m from
1 to 4096 rows against n = 1024 to 11008 columns and k = 1024 to 8192 -- the
4096^3, prefill 512x11008x4096 and single-row 1x4096x4096 products and 33
seeded ones in the first; 8x4096x4096, 2048x11008x4096 and 16 of another
seed, with no size of the first, in the second.  "extra" (fitted too) and
"extra_heldout" (both fitted too) and "extra_heldout2": 1-D convolutions
(H = 1, windows 1x3, 1x5 and 1x7) and products whose rows are not 16-byte
aligned (odd k, row strides + 13), ten of each per set from three seeds,
none of the sizes the benchmark times.

    python3 -m fp32_blocked_gemm_amd.choice_sweep [--set fit|heldout|large|large_heldout] [--mode fast|exact]
        [--only3x3] [--variants 26,27,28] [--out FILE] [--quick]

prints one JSON line per shape (times in us) and a summary line.
"""
import argparse
import json
import random
import sys


def large_products(which):
    """(m, n, k, row-stride padding) of the "large" or "large_heldout" set:
    products of at most 2 * 4096^3 multiply-adds, none of the second in the
    first."""
    def draw(seed, count, first):
        rng, out = random.Random(seed), list(first)
        while len(out) < count:
            m, n, k = (rng.choice([1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 3072, 4096]),
                       rng.choice([1024, 2048, 4096, 8192, 11008]), rng.choice([1024, 2048, 4096, 8192]))
            p = (m, n, k, rng.choice([0, 4]))
            if m * n * k <= 2 * 4096 ** 3 and p not in out:
                out.append(p)
        return out

    fit = draw(41, 36, [(4096, 4096, 4096, 0), (512, 11008, 4096, 0), (1, 4096, 4096, 0)])
    if which == "large":
        return fit
    held = draw(43, 40, [(8, 4096, 4096, 0), (2048, 11008, 4096, 0)])
    return [p for p in held if p[:3] not in {q[:3] for q in fit}][:18]


def extra_shapes(which, synth):
    """1-D convolutions and unaligned products of the "extra" or
    "extra_heldout" set (none of the benchmark's own sizes)."""
    rng = random.Random({"extra": 51, "extra_heldout": 53}.get(which, 57))
    convs, prods = [], []
    while len(convs) < 10:
        n, c, co = rng.choice([1, 2, 4, 8]), rng.choice([64, 128, 256, 384, 512]), rng.choice([64, 128, 256, 512])
        w, kw = rng.choice([512, 1024, 2048, 3000, 8192]), rng.choice([3, 5, 7])
        if (n, c, w, co, kw) == (8, 512, 4096, 512, 5) or n * c * w * co * kw > 2 ** 34:
            continue
        convs.append(synth.ConvShape(f"c1d_{n}_{c}_{w}_{co}_{kw}", n, c, 1, w, co, 1, kw, (1, 1),
                                     (0, kw // 2, 0, kw // 2)))
    while len(prods) < 10:
        m, n, k = rng.choice([100, 333, 700, 1000, 1500, 2500]), rng.choice([250, 777, 1200, 2000]), \
            rng.choice([301, 777, 1531, 2047, 3001])
        if (m, n, k) != (1000, 777, 1531):
            prods.append((m, n, k, 13))
    return convs, prods


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--out", default=None, help="also write the lines to this file")
    ap.add_argument("--set", default="heldout", choices=("fit", "heldout", "large", "large_heldout", "extra", "extra_heldout", "extra_heldout2"))
    ap.add_argument("--quick", action="store_true", help="the first ResNet-50 batch only, 6 products")
    ap.add_argument("--mode", default="fast", choices=("fast", "exact"))
    ap.add_argument("--only3x3", action="store_true", help="3x3 convolutions only")
    ap.add_argument("--variants", default=None,
                    help="comma-separated variants to time besides 0 (default: every one that runs the shape)")
    args = ap.parse_args()
    only = [int(v) for v in args.variants.split(",")] if args.variants else None
    import torch

    import synth
    import bench
    import fp32_blocked_gemm_amd as og

    timer = bench.Timer(torch)
    out = open(args.out, "w") if args.out else None

    def emit(e):
        line = json.dumps(e)
        print(line, flush=True)
        if out:
            out.write(line + "\n")
            out.flush()

    def t_of(call):
        g = timer.graph(lambda: [call() for _ in range(10)])
        # one untimed replay first: the first launches of a kernel after a
        # change of shape or variant ran up to 9 % slower (measured)
        g.replay()
        torch.cuda.synchronize()
        ms = timer.spike(g.replay, min_ms=10.0, reps=3) / 10
        del g
        return round(ms * 1e3, 2)

    # variants that run a shape: every tile variant (exact mode runs 14..16
    # as others and refuses none), and the kernels of their own forms where
    # the shape is theirs (the panel kernel in fast mode only)
    tiles = list(range(1, 18)) + [20]
    if args.mode == "exact":
        tiles = [v for v in tiles if v not in (14, 15, 16)]
    panel = [29, 30] if args.mode == "fast" else []

    def keep(vs):
        return [v for v in vs if only is None or v in only]

    def conv_variants(s):
        if s.Cin // s.groups == 1:
            return None  # depthwise: its own kernel only
        if args.only3x3 and not (s.KH == 3 and s.KW == 3):
            return None
        v = list(tiles)
        if s.KH == 3 and s.KW == 3:
            v += [26, 27, 28, 31, 32, 33]
        if s.KH == 1 and s.KW == 1:
            v += panel
        return keep(v)

    regrets = []

    def run_conv(s, tag):
        vs = conv_variants(s)
        if vs is None:
            return
        x, w = synth.conv_inputs(s, 1)
        dx, dw = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
        y = og.conv2d(dx, dw, stride=s.stride, pad=s.pad, dil=s.dil, groups=s.groups)
        e = {"set": tag, "kind": "conv", "shape": repr(s),
             "dims": [s.N, s.Cin, s.H, s.W, s.Cout, s.KH, s.KW, list(s.stride), list(s.pad), list(s.dil), s.groups]}
        for v in [0] + vs:
            og.set_variant(v)
            e[str(v)] = t_of(lambda: og.conv2d(dx, dw, stride=s.stride, pad=s.pad, dil=s.dil,
                                               groups=s.groups, mode=args.mode, out=y))
        og.set_variant(0)
        best = min(e[str(v)] for v in [0] + vs)
        e["best"] = min(([0] + vs), key=lambda v: e[str(v)])
        e["regret"] = round(e["0"] / best, 4)
        regrets.append(e["regret"])
        emit(e)

    def run_gemm(m, n, k, ld, tag):
        A = torch.randn(m, k + ld, device="cuda")[:, :k]
        B = torch.randn(k, n + ld, device="cuda")[:, :n]
        C = torch.empty(m, n + ld, device="cuda")[:, :n]
        if args.only3x3:
            return
        vs = keep(tiles + panel)
        e = {"set": tag, "kind": "gemm", "shape": f"{m}x{n}x{k} row strides +{ld}", "dims": [m, n, k, ld]}
        for v in [0] + vs:
            og.set_variant(v)
            e[str(v)] = t_of(lambda: og.gemm(A, B, args.mode, out=C))
        og.set_variant(0)
        best = min(e[str(v)] for v in [0] + vs)
        e["best"] = min(([0] + vs), key=lambda v: e[str(v)])
        e["regret"] = round(e["0"] / best, 4)
        regrets.append(e["regret"])
        emit(e)

    products = []
    if args.set.startswith("extra"):
        resnet_b, mobile_b, seeds = (), (), ()
        other, products = extra_shapes(args.set, synth)
    elif args.set in ("large", "large_heldout"):
        resnet_b, mobile_b, other, seeds = (), (), (), ()
        products = large_products(args.set)
    elif args.set == "fit":
        resnet_b, mobile_b, seeds = (1, 2, 3, 4, 5, 6, 8, 12, 16), (1, 2, 4, 6, 8), ((7, 48), (23, 24))
        other = (synth.ConvShape("inc96_35", 8, 96, 35, 35, 96, 3, 3, (1, 1), (1, 1, 1, 1)),
                 synth.ConvShape("inc192_17", 8, 192, 17, 17, 192, 3, 3, (1, 1), (1, 1, 1, 1)),
                 synth.ConvShape("vgg64_112", 1, 64, 112, 112, 64, 3, 3, (1, 1), (1, 1, 1, 1)),
                 synth.ConvShape("u128_32_b4", 4, 128, 32, 32, 128, 3, 3, (1, 1), (1, 1, 1, 1)),
                 synth.ConvShape("vgg128_56_b2", 2, 128, 56, 56, 128, 3, 3, (1, 1), (1, 1, 1, 1)),
                 synth.ConvShape("u256_16_b8", 8, 256, 16, 16, 256, 3, 3, (1, 1), (1, 1, 1, 1)),
                 synth.ConvShape("s2_96_40_b4", 4, 96, 40, 40, 192, 3, 3, (2, 2), (1, 1, 1, 1)),
                 synth.ConvShape("u384_10_b16", 16, 384, 10, 10, 384, 3, 3, (1, 1), (1, 1, 1, 1)),
                 synth.ConvShape("u160_20_b4", 4, 160, 20, 20, 160, 3, 3, (1, 1), (1, 1, 1, 1)),
                 synth.ConvShape("u48_64_b2", 2, 48, 64, 64, 96, 3, 3, (1, 1), (1, 1, 1, 1)),
                 synth.ConvShape("s2_320_24_b8", 8, 320, 24, 24, 320, 3, 3, (2, 2), (1, 1, 1, 1)),
                 synth.ConvShape("u512_12_b2", 2, 512, 12, 12, 256, 3, 3, (1, 1), (1, 1, 1, 1)))
    else:
        resnet_b, mobile_b, seeds = (7, 10), (3, 5), ((31, 24),)
        other = (synth.ConvShape("u80_30_b6", 6, 80, 30, 30, 80, 3, 3, (1, 1), (1, 1, 1, 1)),
                 synth.ConvShape("u224_14_b4", 4, 224, 14, 14, 448, 3, 3, (1, 1), (1, 1, 1, 1)),
                 synth.ConvShape("s2_64_80_b2", 2, 64, 80, 80, 128, 3, 3, (2, 2), (1, 1, 1, 1)),
                 synth.ConvShape("u32_96_b1", 1, 32, 96, 96, 32, 3, 3, (1, 1), (1, 1, 1, 1)))
    if args.quick:
        resnet_b, mobile_b, other = resnet_b[:1], (), ()
        seeds, products = ((seeds[0][0], 6),) if seeds else (), products[:3]
    seen = set()
    for b in resnet_b:
        for s in synth.resnet50_convs(b):
            key = (s.N, s.Cin, s.H, s.Cout, s.KH, s.stride)
            if key not in seen:
                seen.add(key)
                run_conv(s, f"resnet50_b{b}")
    for b in mobile_b:
        for s in synth.mobilenetv3_large_convs(b):
            key = (s.N, s.Cin, s.H, s.Cout, s.KH, s.stride, s.groups)
            if key not in seen:
                seen.add(key)
                run_conv(s, f"mobilenetv3_b{b}")
    for s in other:
        run_conv(s, "conv1d" if args.set.startswith("extra") else "other3x3")
    for m, n, k, ld in products:
        run_gemm(m, n, k, ld, args.set + "_products")
    for seed, nprod in seeds:
        rng = random.Random(seed)
        for _ in range(nprod):
            run_gemm(rng.choice([48, 96, 200, 333, 640, 1200, 2048]), rng.choice([100, 250, 700, 1500, 2900]),
                     rng.choice([64, 300, 777, 1500, 2300]), rng.choice([0, 1, 4]), "random_products")
    regrets.sort()
    n = len(regrets)
    summ = {"summary": True, "shapes": n, "mean_regret": round(sum(regrets) / n, 4),
            "median_regret": regrets[n // 2], "max_regret": regrets[-1],
            "over_5pct": sum(r > 1.05 for r in regrets), "over_10pct": sum(r > 1.10 for r in regrets)}
    emit(summ)
    if out:
        out.close()


if __name__ == "__main__":
    sys.path.insert(0, __import__("os").path.dirname(__import__("os").path.dirname(__import__("os").path.abspath(__file__))))
    main()
