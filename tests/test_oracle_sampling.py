"""Pins of the oracle's row/column sampling and bias paths.

The full-size GPU parity tests compare sampled output rows and longitudes
with `oracle.forward(..., rows=R, cols_out=C)`, and the bias tests with
`bias=b`.  Those arguments only restrict which outputs are evaluated (and add
the layer's per-output-channel bias once, the `bias` parameter of the
DiscreteContinuousConvS2 page): so the sampled result must equal the full
forward pass, which the brute-force and closed-form pins fix, sliced at
[R][..., C], plus b[co] on every output of channel co.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import Desc
from disco_workloads import WORKLOADS, Workload, draw_inputs


def _case(name):
    if name == "c1":
        return WORKLOADS["c1"]
    if name == "stride2_grouped":
        # longitude stride 2, two groups, channel counts that differ per side
        return Workload(name, 7, 2, 6, 4, 2, 33, 64, 17, 32, (3, 3), 7, 4 * math.pi / 16, "f32")
    # anisotropic basis with nphi = 3 (not mirror-symmetric), stride 1
    return Workload(name, 8, 1, 3, 5, 1, 25, 48, 25, 48, (3, 3), 7, 0.45, "f32")


def _desc(wl):
    return Desc(wl.nlat_in, wl.nlon_in, wl.nlat_out, wl.nlon_out, wl.kernel_shape, wl.theta_cutoff)


@pytest.mark.parametrize("name", ["c1", "stride2_grouped", "aniso"])
def test_sampled_forward_equals_sliced_full_forward(name):
    wl = _case(name)
    d = _desc(wl)
    x, w = draw_inputs(wl)
    csr = oracle.psi(d)
    full = oracle.forward(d, x, w, wl.groups, csr=csr)
    rng = np.random.default_rng(3)
    rows = sorted({0, 1, wl.nlat_out // 2, wl.nlat_out - 1}
                  | set(rng.choice(wl.nlat_out, 3, replace=False).tolist()))
    cols = sorted({0, wl.nlon_out - 1} | set(rng.choice(wl.nlon_out, 5, replace=False).tolist()))
    bias = rng.standard_normal(wl.Co)
    got = oracle.forward(d, x, w, wl.groups, csr=csr, rows=rows, cols_out=cols, bias=bias)
    want = full[:, :, rows][:, :, :, cols] + bias[None, :, None, None]
    assert got.shape == (wl.B, wl.Co, len(rows), len(cols))
    scale = np.max(np.abs(want))
    assert np.max(np.abs(got - want)) <= 1e-13 * scale
    # without a csr the rows are rebuilt one by one: same values
    got2 = oracle.forward(d, x, w, wl.groups, rows=rows, cols_out=cols, bias=bias)
    assert np.max(np.abs(got2 - want)) <= 1e-13 * scale


@pytest.mark.parametrize("name", ["c1", "stride2_grouped", "aniso"])
def test_sampled_contraction_equals_sliced_full_contraction(name):
    wl = _case(name)
    d = _desc(wl)
    x, _ = draw_inputs(wl)
    csr = oracle.psi(d)
    full = oracle.contract(d, x, csr=csr)
    rows = [wl.nlat_out - 1, 0, wl.nlat_out // 3]          # any order, repeats allowed
    cols = [wl.nlon_out - 1, 0, 0, wl.nlon_out // 2]
    got = oracle.contract(d, x, csr=csr, rows=rows, cols_out=cols)
    want = full[:, :, :, rows][:, :, :, :, cols]
    # same support points added in the same order for every output: exact
    assert np.array_equal(got, want)


def test_bias_is_added_once_per_output_channel():
    wl = _case("stride2_grouped")
    d = _desc(wl)
    x, w = draw_inputs(wl)
    csr = oracle.psi(d)
    bias = np.arange(1, wl.Co + 1, dtype=np.float64) * 10.0
    a = oracle.forward(d, x, w, wl.groups, csr=csr)
    b = oracle.forward(d, x, w, wl.groups, csr=csr, bias=bias)
    diff = b - a
    for co in range(wl.Co):
        assert np.allclose(diff[:, co], bias[co], rtol=0, atol=1e-12)
    # a zero input gives exactly the bias everywhere
    z = oracle.forward(d, np.zeros_like(x), w, wl.groups, csr=csr, bias=bias)
    assert np.array_equal(z, np.broadcast_to(bias[None, :, None, None], z.shape))
