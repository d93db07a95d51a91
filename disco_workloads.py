"""Seeded synthetic workloads for the forward DISCO convolution on the 2-sphere.

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It holds configuration metadata and random-number draws only: no geometry, no
quadrature, no basis functions and no contraction.  Both the HIP path and the
oracle receive the arrays it returns.

The five workloads follow the problem statement of the DISCO layer
(torch_harmonics.DiscreteContinuousConvS2 page, forward equation and parameter
list: (batch, channels, nlat, nlon) tensors, kernel_shape, theta_cutoff,
equiangular grids, groups).  Shapes, dtypes and value distributions are the
synthetic benchmark cases this project is measured on:

* x ~ N(0, 1), drawn first, as float32, shape [B, Ci, nlat_in, nlon_in];
* w ~ N(0, 1 / ((Ci/groups) * K)), shape [Co, Ci/groups, K];
* bf16 cases round both to bfloat16 with round-to-nearest-even;
* numpy.random.default_rng(seed), seed = case number.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    Ci: int
    Co: int
    groups: int
    nlat_in: int
    nlon_in: int
    nlat_out: int
    nlon_out: int
    kernel_shape: tuple          # (nr,) isotropic or (nr, nphi) anisotropic
    K: int                       # number of basis functions for kernel_shape
    theta_cutoff: float          # radians
    dtype: str                   # "f32" or "bf16" (inputs and weights)
    note: str = field(default="")

    @property
    def out_points_cout(self) -> int:
        """Output points times output channels of one forward call."""
        return self.B * self.nlat_out * self.nlon_out * self.Co


WORKLOADS = {
    "c1": Workload("c1", 1, 1, 4, 4, 1, 33, 64, 33, 64, (3,), 3,
                   4 * math.pi / 32, "f32", "tiny isotropic case"),
    "c2": Workload("c2", 2, 4, 32, 32, 1, 129, 256, 129, 256, (3, 3), 7,
                   4 * math.pi / 128, "f32", "anisotropic, fp32"),
    "c3": Workload("c3", 3, 2, 64, 64, 1, 361, 720, 181, 360, (3, 3), 7,
                   4 * math.pi / 180, "bf16", "downsampling, longitude stride 2"),
    "c4": Workload("c4", 4, 1, 128, 128, 1, 721, 1440, 721, 1440, (3, 3), 7,
                   4 * math.pi / 720, "bf16", "full-resolution 0.25 degree grid"),
    "c5": Workload("c5", 5, 1, 256, 256, 256, 721, 1440, 361, 720, (5, 4), 17,
                   6 * math.pi / 360, "f32", "depthwise, downsampling"),
}

HEADLINE = "c4"


def draw_inputs(wl: Workload, seed: int | None = None):
    """Return (x, w) as float32 numpy arrays for workload `wl`.

    x is drawn before w from one generator.  Rounding to bfloat16 for bf16
    cases is done by `round_bf16`, not here, so that both sides of a parity
    test can see the same float32 draw.
    """
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    x = rng.standard_normal((wl.B, wl.Ci, wl.nlat_in, wl.nlon_in), dtype=np.float32)
    std = 1.0 / math.sqrt((wl.Ci // wl.groups) * wl.K)
    w = (rng.standard_normal((wl.Co, wl.Ci // wl.groups, wl.K), dtype=np.float32)
         * np.float32(std)).astype(np.float32)
    return x, w


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the rounded values widened back to float32, so that numpy code can
    consume them; `bf16_bits` gives the raw 16-bit patterns.
    """
    bits = bf16_bits(a).astype(np.uint32) << 16
    return bits.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float32 `a`, round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    nan = np.isnan(a)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def small_variant(wl: Workload, nlat_in: int, nlon_in: int, nlat_out: int,
                  nlon_out: int, B: int | None = None, Ci: int | None = None,
                  Co: int | None = None, groups: int | None = None,
                  theta_cutoff: float | None = None) -> Workload:
    """A reduced copy of `wl` with other grid sizes (for fast parity tests).

    When theta_cutoff is not given it keeps the workload's ratio of cutoff to
    the output latitude spacing.
    """
    if theta_cutoff is None:
        ratio = wl.theta_cutoff / (math.pi / (wl.nlat_out - 1))
        theta_cutoff = ratio * math.pi / (nlat_out - 1)
    return Workload(wl.name + "_small", wl.seed, B or wl.B, Ci or wl.Ci,
                    Co or wl.Co, groups or wl.groups, nlat_in, nlon_in,
                    nlat_out, nlon_out, wl.kernel_shape, wl.K, theta_cutoff,
                    wl.dtype, "reduced grid of " + wl.name)
