"""Seeded synthetic inputs for the tests, the smoke check and the benchmark.

This module holds none of the engine's arithmetic: it draws numbers with
numpy's PCG64 generator and stores them in the operand formats through
torch's CPU casts (float32 -> float16 / bfloat16 / float8_e4m3fn /
float8_e5m2, round to nearest even).  Both the HIP path and the CPU oracle read the same stored
codes.

Seeds: workload ``i`` (1..5) uses base seed ``1000 + i``; its operand streams
are ``10 * base + 0`` (A, or dY for wgrad), ``+1`` (B, or X), ``+2`` (per-row
scale of A) and ``+3`` (per-column scale of B).
"""

from dataclasses import dataclass

import numpy as np
import torch

TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn,
            "e5m2": torch.float8_e5m2, "f32": torch.float32}
CODE_DT = {"f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8, "e5m2": np.uint8,
           "f32": np.uint32}


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def draw(dist, n, seed):
    """float64 draws: ``uniform`` U[-1, 1], ``normal`` N(0, 1), ``normal01``
    N(0, 1) * 0.1, ``scale`` U[0.5, 2]."""
    g = rng(seed)
    if dist == "uniform":
        return g.uniform(-1.0, 1.0, n)
    if dist == "normal":
        return g.standard_normal(n)
    if dist == "normal01":
        return g.standard_normal(n) * 0.1
    if dist == "scale":
        return g.uniform(0.5, 2.0, n)
    raise ValueError(dist)


def to_codes(values, fmt):
    """Store float values in ``fmt`` via torch's CPU cast; returns the codes."""
    t = torch.from_numpy(np.ascontiguousarray(values, dtype=np.float32)).to(TORCH_DT[fmt])
    view = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[np.dtype(CODE_DT[fmt]).itemsize]
    return t.view(view).numpy().view(CODE_DT[fmt])


def integer_codes(fmt, n, seed, density, vmax=2):
    """Sparse small integers in [-vmax, vmax]: every product and partial sum
    of such operands is exact in fp32."""
    g = rng(seed)
    v = g.integers(-vmax, vmax + 1, n).astype(np.float64)
    v = np.where(g.random(n) < density, v, 0.0)
    return to_codes(v, fmt)


def pow2_scales(n, seed, lo=-2, hi=2):
    """Power-of-two scales (products with them stay exact)."""
    return (2.0 ** rng(seed).integers(lo, hi + 1, n)).astype(np.float32)


@dataclass
class GemmWorkload:
    index: int
    name: str
    M: int
    N: int
    K: int
    dtype_ab: str
    dtype_c: str
    dist: str
    tile: str
    modes: tuple
    reductions: tuple
    ctas: int
    scales: bool = False
    op: str = "gemm"
    scale_mode: str = "rowcol"   # "tensor": one scale per operand; "mx": E8M0 block scales

    @property
    def seed(self):
        return 1000 + self.index

    def flops(self):
        return 2.0 * self.M * self.N * self.K

    def inputs(self):
        """dict with A (M*K codes), B (N*K codes, column-major), optional
        scale_a / scale_b float32 vectors."""
        s = self.seed * 10
        out = {
            "A": to_codes(draw(self.dist, self.M * self.K, s + 0), self.dtype_ab),
            "B": to_codes(draw(self.dist, self.N * self.K, s + 1), self.dtype_ab),
        }
        if self.scales and self.scale_mode == "mx":
            # E8M0 block scales 2^-3 .. 2^3, one per 32 K elements of a row
            # of A / a column of B.
            nb = self.K // 32
            out["scale_a"] = (127 + rng(s + 2).integers(-3, 4, self.M * nb)).astype(np.uint8)
            out["scale_b"] = (127 + rng(s + 3).integers(-3, 4, self.N * nb)).astype(np.uint8)
        elif self.scales:
            per = self.scale_mode == "rowcol"
            out["scale_a"] = draw("scale", self.M if per else 1, s + 2).astype(np.float32)
            out["scale_b"] = draw("scale", self.N if per else 1, s + 3).astype(np.float32)
        return out


@dataclass
class WgradWorkload:
    index: int
    name: str
    n: int
    h: int
    w: int
    c: int
    k: int
    r: int
    s: int
    stride: tuple
    pad: tuple
    groups: int
    dtype: str
    dist: str
    tile: str
    modes: tuple
    reductions: tuple
    ctas: int
    op: str = "wgrad"

    @property
    def seed(self):
        return 1000 + self.index

    @property
    def out_hw(self):
        ho = (self.h + 2 * self.pad[0] - self.r) // self.stride[0] + 1
        wo = (self.w + 2 * self.pad[1] - self.s) // self.stride[1] + 1
        return ho, wo

    def flops(self):
        ho, wo = self.out_hw
        return 2.0 * self.k * (self.c // self.groups) * self.r * self.s * self.n * ho * wo

    def inputs(self):
        ho, wo = self.out_hw
        s = self.seed * 10
        return {
            "dy": to_codes(draw(self.dist, self.n * ho * wo * self.k, s + 0), self.dtype),
            "x": to_codes(draw(self.dist, self.n * self.h * self.w * self.c, s + 1), self.dtype),
        }


@dataclass
class ConvWorkload:
    """Forward convolution (op "fwd": act = X, out = Y) or its input gradient
    (op "dgrad": act = dY, out = dX) of one layer; filt is the KRSC filter."""
    index: int
    name: str
    op: str
    n: int
    h: int
    w: int
    c: int
    k: int
    r: int
    s: int
    stride: tuple
    pad: tuple
    groups: int
    dtype: str
    dtype_out: str
    dist: str
    tile: str
    modes: tuple
    reductions: tuple
    ctas: int

    @property
    def seed(self):
        return 1000 + self.index

    @property
    def out_hw(self):
        ho = (self.h + 2 * self.pad[0] - self.r) // self.stride[0] + 1
        wo = (self.w + 2 * self.pad[1] - self.s) // self.stride[1] + 1
        return ho, wo

    def flops(self):
        """Algorithmic FLOPs of the layer (the same for both ops)."""
        ho, wo = self.out_hw
        return 2.0 * self.n * ho * wo * self.k * self.r * self.s * (self.c // self.groups)

    def inputs(self):
        ho, wo = self.out_hw
        s = self.seed * 10
        na = self.n * self.h * self.w * self.c if self.op == "fwd" else self.n * ho * wo * self.k
        return {
            "act": to_codes(draw(self.dist, na, s + 0), self.dtype),
            "filt": to_codes(draw(self.dist, self.k * self.r * self.s * (self.c // self.groups),
                                  s + 1), self.dtype),
        }


# The five workloads.  Tiles for 1 and 2 are the ones the workloads name;
# 3, 4 and 5 use the tiles measured fastest for them (4: block-diagonal,
# below).  Workload 3
# runs 256x256 tiles (9 output tiles) over a pool of 252 = 9 x 28 CTAs: every
# stream-K CTA then holds 56 whole iterations of one tile, which the k-major
# CTA order turns into 28 k ranges read by all 9 tiles at about the same time.
# Workloads 3 and 4 hand their tiles on with the reduce-scatter fix-up: the
# linear fix-up's additions in the linear order, split over the tile's
# contributors (its results are the linear fix-up's bit for bit).
WORKLOADS = {
    1: GemmWorkload(1, "gemm_f16_256x256x4096_pool6_linear", 256, 256, 4096, "f16", "f16",
                    "uniform", "128x128x32", ("dp_sk",), ("linear",), 6),
    2: GemmWorkload(2, "gemm_bf16_4864x4096x4096_tree", 4864, 4096, 4096, "bf16", "bf16",
                    "normal01", "256x256x64", ("persistent", "dp_sk"), ("tree",), 256),
    3: WgradWorkload(3, "wgrad_f16_n32_56x56_c256_k256_3x3", 32, 56, 56, 256, 256, 3, 3,
                     (1, 1), (1, 1), 1, "f16", "uniform", "256x256x64",
                     ("persistent", "dp_sk"), ("scatter", "tree", "linear", "atomic", "workspace"),
                     252),
    # 16 channels per group: the block-diagonal tile (four whole groups per
    # 64-row tile, whole 128-byte lines) over 224 CTAs, i.e. 28 whole slices
    # of 14 iterations per tile, with the reduce-scatter fix-up; the
    # per-group 32x64x64 tile and the one-CTA linear fold are reported
    # beside it.
    4: WgradWorkload(4, "wgrad_bf16_n64_28x28_c512_k512_g32_3x3_s2", 64, 28, 28, 512, 512, 3, 3,
                     (2, 2), (1, 1), 32, "bf16", "uniform", "64x144x32", ("dp_sk",), ("scatter",),
                     224),
    5: GemmWorkload(5, "gemm_e4m3_8192x8192x8192_rowcol_scales", 8192, 8192, 8192, "e4m3",
                    "bf16", "normal", "256x256x128", ("persistent",), ("workspace",), 256,
                    scales=True),
}

# Workloads of the rows built after the five: the other two convolutions of
# the two wgrad layers (forward and input gradient), on the same engine, in
# the launches measured fastest (256x256x64 tiles, persistent, tree fix-up
# for the dense layer; the block-diagonal 128x64x32 tile for the grouped
# one, 16 channels per group, two CTAs per CU, where a tile's reduction is
# 5 MAC iterations (dgrad: 1 or 2, its tiles run stride phase by phase) and
# stream-K does not pay), and the
# fp8 GEMM of workload 5 with OCP MX (E8M0) block scales instead of
# row/column scales (256x256x128 tiles: 4 ring slots once the scale bytes
# ride along, refilled among the MFMAs).
NEXT_WORKLOADS = {
    6: ConvWorkload(6, "fwd_f16_n32_56x56_c256_k256_3x3", "fwd", 32, 56, 56, 256, 256, 3, 3,
                    (1, 1), (1, 1), 1, "f16", "f16", "uniform", "256x256x64", ("persistent",),
                    ("tree",), 256),
    7: ConvWorkload(7, "dgrad_f16_n32_56x56_c256_k256_3x3", "dgrad", 32, 56, 56, 256, 256, 3, 3,
                    (1, 1), (1, 1), 1, "f16", "f16", "uniform", "256x256x64", ("persistent",),
                    ("tree",), 256),
    8: ConvWorkload(8, "fwd_bf16_n64_28x28_c512_k512_g32_3x3_s2", "fwd", 64, 28, 28, 512, 512, 3,
                    3, (2, 2), (1, 1), 32, "bf16", "bf16", "uniform", "128x64x32", ("dp",),
                    ("tree",), 512),
    9: ConvWorkload(9, "dgrad_bf16_n64_28x28_c512_k512_g32_3x3_s2", "dgrad", 64, 28, 28, 512, 512,
                    3, 3, (2, 2), (1, 1), 32, "bf16", "bf16", "uniform", "128x64x32", ("persistent",),
                    ("tree",), 512),
    10: GemmWorkload(10, "gemm_e4m3_8192x8192x8192_mx_e8m0", 8192, 8192, 8192, "e4m3", "bf16",
                     "normal", "256x256x128", ("persistent",), ("workspace",), 256, scales=True,
                     scale_mode="mx"),
}

# Further launches of a workload reported beside its own: the dense wgrad
# layer with the tree fix-up (its own launch takes the reduce-scatter
# fix-up; all five run at full size in the parity tests); the
# grouped layer with the linear and tree fix-ups on the block-diagonal tile
# and with the per-group tile (partial 32-row M tiles, groups folded into
# GEMM-M one per tile); the grouped forward and dgrad on the dense
# per-group 128x128x64 tile (16 of its 128 columns used).
EXTRA_LAUNCHES = {3: [("256x256x64", "persistent", "tree", 252)],
                  4: [("64x144x32", "dp_sk", "tree", 224), ("64x144x32", "dp_sk", "linear", 128),
                      ("32x64x64", "dp_sk", "linear", 512)],
                  8: [("128x64x32", "persistent", "tree", 512), ("128x128x64", "dp_sk", "tree", 256)],
                  9: [("128x128x64", "dp_sk", "tree", 256)]}

# Earlier name of the first four of them.
LAYER_WORKLOADS = {i: w for i, w in NEXT_WORKLOADS.items() if i in (6, 7, 8, 9)}
