"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds none of the method's arithmetic: only random draws, buffer
layouts (row strides with gaps, sentinels), the injection of special values
and the shape tables of the workloads.  Both the GPU path and the oracle are
fed from here; neither is imported here.

Workloads (sizes from the matrix-product and convolution workloads these
kernels are measured on):
  * square fp32 GEMM 256^3, uniform[-1,1], one generator seeded 0 drawing A
    then B;
  * 4096^3 and the ragged 1000x777x1531 with row strides dim+13, N(0,1) with
    0.1% special values at seeded positions (plus clean copies);
  * prefill-shaped 512x4096 * 4096x11008 (activations N(0,1), weights
    N(0,0.02)) and the skinny 1x4096 * 4096x4096;
  * the 53 convolutions of ResNet-50 v1.5 at 224x224, batch 1 and 8, inputs
    N(0,1), He-normal weights;
  * a grouped, dilated, strided convolution and a 1-D convolution run as H=1.
"""
from __future__ import annotations

import math

import numpy as np

# Bit patterns written into the gaps of row-strided buffers.  The input gap
# value is a NaN with a payload, so a read of a gap shows up in the results;
# the output gap value is an ordinary number that must survive a call.
GAP_IN_BITS = 0x7FA5A5A5
GAP_OUT_BITS = 0x5A5A5A5A

# NaN inputs: canonical, negative, with payload, signalling.
NAN_BITS = (0x7FC00000, 0xFFC00000, 0x7FC12345, 0x7F800001)


def seed_for(config: int, tensor: int) -> int:
    """Seed of tensor `tensor` of workload number `config`."""
    return 1000 * config + tensor


def uniform(shape, seed: int, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    return np.random.default_rng(seed).uniform(lo, hi, size=shape).astype(np.float32)


def normal(shape, seed: int, std: float = 1.0) -> np.ndarray:
    g = np.random.default_rng(seed)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def strided(values: np.ndarray, ld: int, gap_bits: int = GAP_IN_BITS):
    """Copy a (rows, cols) matrix into a (rows, ld) buffer whose gaps hold `gap_bits`.

    Returns (buffer, view): the view is the logical matrix inside the buffer.
    """
    rows, cols = values.shape
    assert ld >= max(1, cols)
    buf = np.empty((rows, ld), np.float32)
    buf.view(np.uint32)[...] = np.uint32(gap_bits)
    view = buf[:, :cols]
    view[...] = values
    return buf, view


def inject_specials(view: np.ndarray, frac: float, seed: int) -> int:
    """Overwrite a fraction of the elements of `view` with special values.

    Positions are drawn without replacement from a generator seeded `seed`;
    the classes come in equal shares: NaN (the four patterns of NAN_BITS in
    turn), +inf, -inf, subnormal (random sign, random non-zero 23-bit
    fraction) and -0.  Returns the number of elements changed.
    """
    g = np.random.default_rng(seed)
    rows, cols = view.shape
    total = rows * cols
    count = int(round(frac * total))
    if count == 0:
        return 0
    pos = g.choice(total, size=count, replace=False)
    cls = np.arange(count) % 5
    bits = np.empty(count, np.uint32)
    nan_pick = (np.arange(count) // 5) % len(NAN_BITS)
    bits[cls == 0] = np.array(NAN_BITS, np.uint32)[nan_pick[cls == 0]]
    bits[cls == 1] = 0x7F800000
    bits[cls == 2] = 0xFF800000
    n_sub = int((cls == 3).sum())
    frac_bits = g.integers(1, 1 << 23, size=n_sub, dtype=np.uint32)
    sign_bits = g.integers(0, 2, size=n_sub, dtype=np.uint32) << np.uint32(31)
    bits[cls == 3] = frac_bits | sign_bits
    bits[cls == 4] = 0x80000000
    u = view.view(np.uint32)
    u[pos // cols, pos % cols] = bits
    return count


# ---------------------------------------------------------------------------
# Matrix-product workloads
# ---------------------------------------------------------------------------

class GemmCase:
    """Inputs of one matrix product: strided buffers plus their logical views."""

    def __init__(self, name, m, n, k, lda, ldb, ldc, A, B):
        self.name, self.m, self.n, self.k = name, m, n, k
        self.lda, self.ldb, self.ldc = lda, ldb, ldc
        self.A_buf, self.A = strided(A, lda) if m > 0 else (A, A)
        self.B_buf, self.B = strided(B, ldb) if k > 0 else (B, B)

    def new_c(self) -> tuple[np.ndarray, np.ndarray]:
        buf = np.empty((self.m, self.ldc), np.float32)
        buf.view(np.uint32)[...] = np.uint32(GAP_OUT_BITS)
        return buf, buf[:, :self.n]

    @property
    def flops(self) -> float:
        return 2.0 * self.m * self.n * self.k


def gemm_square256() -> GemmCase:
    """m = n = k = 256, row-major, ld = 256, A and B uniform[-1,1] from seed 0."""
    g = np.random.default_rng(0)
    A = g.uniform(-1, 1, size=(256, 256)).astype(np.float32)
    B = g.uniform(-1, 1, size=(256, 256)).astype(np.float32)
    return GemmCase("gemm_256_exact", 256, 256, 256, 256, 256, 256, A, B)


def gemm_normal(name: str, m: int, n: int, k: int, pad: int, config: int,
                specials: float, std_b: float = 1.0) -> GemmCase:
    """N(0,1) A and N(0,std_b) B with row strides dim+pad and optional special values."""
    A = normal((m, k), seed_for(config, 0))
    B = normal((k, n), seed_for(config, 1), std_b)
    c = GemmCase(name, m, n, k, k + pad, n + pad, n + pad, A, B)
    if specials > 0:
        inject_specials(c.A, specials, seed_for(config, 2))
        inject_specials(c.B, specials, seed_for(config, 3))
    return c


def gemm_4096(specials: bool = True) -> GemmCase:
    return gemm_normal("gemm_4096" + ("" if specials else "_clean"), 4096, 4096, 4096, 0, 2,
                       0.001 if specials else 0.0)


def gemm_ragged(specials: bool = True) -> GemmCase:
    return gemm_normal("gemm_1000x777x1531_ld13" + ("" if specials else "_clean"),
                       1000, 777, 1531, 13, 2, 0.001 if specials else 0.0)


def gemm_prefill() -> GemmCase:
    return gemm_normal("gemm_prefill_512x11008x4096", 512, 11008, 4096, 0, 3, 0.0, std_b=0.02)


def gemm_skinny() -> GemmCase:
    return gemm_normal("gemm_skinny_1x4096x4096", 1, 4096, 4096, 0, 3, 0.0, std_b=0.02)


# ---------------------------------------------------------------------------
# Convolution workloads
# ---------------------------------------------------------------------------

class ConvShape:
    """One NCHW convolution: sizes, per-axis stride/pad/dilation and groups."""

    def __init__(self, name, N, Cin, H, W, Cout, KH, KW, stride=(1, 1), pad=(0, 0, 0, 0),
                 dil=(1, 1), groups=1):
        self.name = name
        self.N, self.Cin, self.H, self.W, self.Cout = N, Cin, H, W, Cout
        self.KH, self.KW = KH, KW
        self.stride, self.pad, self.dil, self.groups = tuple(stride), tuple(pad), tuple(dil), groups

    def with_batch(self, N: int) -> "ConvShape":
        return ConvShape(self.name, N, self.Cin, self.H, self.W, self.Cout, self.KH, self.KW,
                         self.stride, self.pad, self.dil, self.groups)

    def __repr__(self):
        return (f"ConvShape({self.name}: N{self.N} {self.Cin}->{self.Cout} {self.H}x{self.W} "
                f"k{self.KH}x{self.KW} s{self.stride} p{self.pad} d{self.dil} g{self.groups})")


def resnet50_convs(batch: int = 1) -> list[ConvShape]:
    """The 53 convolutions of ResNet-50 v1.5 at 224x224, in network order.

    Stem 7x7/2 pad 3; four stages of bottleneck blocks (3, 4, 6, 3) with widths
    64, 128, 256, 512 and expansion 4; the stride sits on the 3x3 convolution
    of a stage's first block, whose 1x1 downsample (stride 1 or 2) follows its
    third convolution.
    """
    layers = [ConvShape("stem", batch, 3, 224, 224, 64, 7, 7, (2, 2), (3, 3, 3, 3))]
    in_ch = 64
    # (blocks, width, spatial size entering the stage, spatial size leaving it)
    stages = ((3, 64, 56, 56), (4, 128, 56, 28), (6, 256, 28, 14), (3, 512, 14, 7))
    for stage, (blocks, width, hw_in, hw_out) in enumerate(stages, start=1):
        out_ch = 4 * width
        for b in range(blocks):
            first = b == 0
            s = hw_in // hw_out if first else 1
            hw = hw_in if first else hw_out
            tag = f"layer{stage}.{b}"
            layers.append(ConvShape(tag + ".c1", batch, in_ch, hw, hw, width, 1, 1))
            layers.append(ConvShape(tag + ".c2", batch, width, hw, hw, width, 3, 3, (s, s),
                                    (1, 1, 1, 1)))
            layers.append(ConvShape(tag + ".c3", batch, width, hw_out, hw_out, out_ch, 1, 1))
            if first:
                layers.append(ConvShape(tag + ".down", batch, in_ch, hw, hw, out_ch, 1, 1,
                                        (s, s)))
            in_ch = out_ch
    assert len(layers) == 53
    return layers


def grouped_dilated() -> ConvShape:
    return ConvShape("grouped_g32_d2_s2", 4, 256, 64, 64, 256, 3, 3, (2, 2), (2, 2, 2, 2),
                     (2, 2), 32)


def conv1d_h1() -> ConvShape:
    """1-D convolution as H = 1: pads only on the width axis."""
    return ConvShape("conv1d_w4096_k5", 8, 512, 1, 4096, 512, 1, 5, (1, 1), (0, 2, 0, 2))


def conv_inputs(shape: ConvShape, seed: int, dist: str = "normal") -> tuple[np.ndarray, np.ndarray]:
    """Input x [N,Cin,H,W] and weights w [Cout,Cin/G,KH,KW] for one convolution.

    dist 'normal': x N(0,1), w He-normal (std sqrt(2/fan_in), fan_in = Cin/G*KH*KW).
    dist 'uniform': both uniform[-1,1].
    """
    xs = (shape.N, shape.Cin, shape.H, shape.W)
    ws = (shape.Cout, shape.Cin // shape.groups, shape.KH, shape.KW)
    if dist == "uniform":
        return uniform(xs, seed), uniform(ws, seed + 1)
    fan_in = ws[1] * ws[2] * ws[3]
    return normal(xs, seed), normal(ws, seed + 1, math.sqrt(2.0 / fan_in))


def mobilenetv3_large_depthwise(batch: int = 1) -> list[ConvShape]:
    """The 15 depthwise convolutions of MobileNetV3-large at 224x224, in order.

    Each bottleneck's depthwise convolution runs over its expanded channels
    (groups = channels, multiplier 1) with a 3x3 or 5x5 window, padding
    window // 2 and stride 1 or 2 (Howard et al. 2019, "Searching for
    MobileNetV3", table 1).
    """
    # (channels, input size, window, stride)
    spec = ((16, 112, 3, 1), (64, 112, 3, 2), (72, 56, 3, 1), (72, 56, 5, 2), (120, 28, 5, 1),
            (120, 28, 5, 1), (240, 28, 3, 2), (200, 14, 3, 1), (184, 14, 3, 1), (184, 14, 3, 1),
            (480, 14, 3, 1), (672, 14, 3, 1), (672, 14, 5, 2), (960, 7, 5, 1), (960, 7, 5, 1))
    out = []
    for i, (c, hw, k, s) in enumerate(spec):
        p = k // 2
        out.append(ConvShape(f"dw{i + 1}", batch, c, hw, hw, c, k, k, (s, s), (p, p, p, p),
                             (1, 1), c))
    return out


def mobilenetv3_large_se(batch: int = 1) -> list[ConvShape]:
    """The 16 squeeze-and-excitation convolutions of MobileNetV3-large, in order.

    Each of the 8 blocks with squeeze-and-excitation pools its C expanded
    channels to 1x1 and runs two 1x1 convolutions, C -> S and S -> C, with S
    the quarter of C rounded up to a multiple of 8 (24, 32, 32, 120, 168,
    168, 240, 240): at batch 1 each is a matrix-vector product.
    """
    out = []
    for i, (c, s) in enumerate(((72, 24), (120, 32), (120, 32), (480, 120), (672, 168),
                                (672, 168), (960, 240), (960, 240))):
        out.append(ConvShape(f"se{i + 1}.reduce", batch, c, 1, 1, s, 1, 1))
        out.append(ConvShape(f"se{i + 1}.expand", batch, s, 1, 1, c, 1, 1))
    return out


def gemm_single_column() -> GemmCase:
    """m = k = 4096, n = 1: a 4096x4096 row-major matrix times one column (N(0,0.02) x N(0,1))."""
    A = normal((4096, 4096), seed_for(3, 10), 0.02)
    B = normal((4096, 1), seed_for(3, 11))
    return GemmCase("gemm_single_column_4096x1x4096", 4096, 1, 4096, 4096, 1, 1, A, B)


def transformer_linear_shapes(model: str) -> list[tuple[str, int, int, int, int]]:
    """The matrix products of one model's linear layers: (name, m, n, k, count).

    m = token rows, k = input features, n = output features; the weights are
    stored as n x k (out x in), so these run as products with an N x K operand.
    Public architecture dimensions: BERT-base (hidden 768, 3072 FFN, 12
    layers), MiniLM-L6 (hidden 384, 1536 FFN, 6 layers), the Whisper-small
    encoder (768, 3072, 12 layers); per layer the query, key, value and output
    projections and the two FFN layers.  Token rows as in the pages' model
    rows: 32 x 128 (and 128) for BERT and MiniLM, 1500 frames for Whisper.
    Attention's own products are left out, as on the pages.
    """
    dims = {"bert_base_4096": (4096, 768, 3072, 12), "bert_base_128": (128, 768, 3072, 12),
            "minilm_l6_4096": (4096, 384, 1536, 6), "whisper_small_enc_1500": (1500, 768, 3072, 12)}
    rows, h, f, layers = dims[model]
    return [("qkvo", rows, h, h, 4 * layers), ("ffn_up", rows, f, h, layers),
            ("ffn_down", rows, h, f, layers)]


def whisper_small_frontend() -> list[ConvShape]:
    """The Whisper-small encoder's two 1-D convolutions over 3000 mel frames
    (80 -> 768, width 3, pad 1; 768 -> 768, width 3, stride 2, pad 1), as H = 1."""
    return [ConvShape("whisper.conv1", 1, 80, 1, 3000, 768, 1, 3, (1, 1), (0, 1, 0, 1)),
            ConvShape("whisper.conv2", 1, 768, 1, 3000, 768, 1, 3, (1, 2), (0, 1, 0, 1))]


def mobilenetv3_large_convs(batch: int = 1) -> list[ConvShape]:
    """The convolutions of MobileNetV3-large at 224x224 without the
    squeeze-and-excitation and classifier layers: the 3x3/2 stem, for each
    bottleneck its 1x1 expansion (when the expanded width differs from the
    input), its depthwise convolution and its 1x1 projection, and the last
    1x1 convolution (160 -> 960) (Howard et al. 2019, table 1)."""
    layers = [ConvShape("stem", batch, 3, 224, 224, 16, 3, 3, (2, 2), (1, 1, 1, 1))]
    # (input channels, window, expanded, output channels, stride, input size)
    spec = ((16, 3, 16, 16, 1, 112), (16, 3, 64, 24, 2, 112), (24, 3, 72, 24, 1, 56),
            (24, 5, 72, 40, 2, 56), (40, 5, 120, 40, 1, 28), (40, 5, 120, 40, 1, 28),
            (40, 3, 240, 80, 2, 28), (80, 3, 200, 80, 1, 14), (80, 3, 184, 80, 1, 14),
            (80, 3, 184, 80, 1, 14), (80, 3, 480, 112, 1, 14), (112, 3, 672, 112, 1, 14),
            (112, 5, 672, 160, 2, 14), (160, 5, 960, 160, 1, 7), (160, 5, 960, 160, 1, 7))
    for i, (cin, k, exp, cout, s, hw) in enumerate(spec):
        tag = f"bneck{i + 1}"
        if exp != cin:
            layers.append(ConvShape(tag + ".expand", batch, cin, hw, hw, exp, 1, 1))
        p = k // 2
        layers.append(ConvShape(tag + ".dw", batch, exp, hw, hw, exp, k, k, (s, s), (p, p, p, p),
                                (1, 1), exp))
        layers.append(ConvShape(tag + ".project", batch, exp, hw // s, hw // s, cout, 1, 1))
    layers.append(ConvShape("last", batch, 160, 7, 7, 960, 1, 1))
    return layers
