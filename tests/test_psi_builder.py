"""The library's host Psi builder (C++) against the oracle (Python), on CPU.

Indices are compared bit for bit; values within 1e-12 of the row's largest
value (both sides are float64 and evaluate the same definition with different
code).  Shares nothing with the oracle but the workload metadata.
"""
import math

import numpy as np
import pytest

import oracle
from disco_workloads import WORKLOADS
import spherical_disco_convolution_amd as sdc


def _pair(nli, nfi, nlo, nfo, ks, cut):
    lib = sdc.psi_build(nli, nfi, nlo, nfo, ks, cut)
    ref = oracle.psi(oracle.Desc(nli, nfi, nlo, nfo, tuple(ks), cut))
    return lib, ref


def _compare(lib, ref):
    row_ptr, in_lat, lon_off, vals = lib.export()
    assert np.array_equal(row_ptr, ref.row_ptr)
    assert np.array_equal(in_lat, ref.in_lat)
    assert np.array_equal(lon_off, ref.lon_off)
    assert vals.shape == ref.vals.shape
    scale = max(1e-300, float(np.max(np.abs(ref.vals))))
    assert np.max(np.abs(vals - ref.vals)) <= 1e-12 * scale


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4", "c5"])
def test_builder_matches_oracle_on_workloads(key):
    wl = WORKLOADS[key]
    lib, ref = _pair(wl.nlat_in, wl.nlon_in, wl.nlat_out, wl.nlon_out, wl.kernel_shape,
                     wl.theta_cutoff)
    _compare(lib, ref)
    assert lib.K == wl.K


@pytest.mark.parametrize("case", [
    (9, 16, 9, 16, (3,), 0.9),
    (17, 32, 9, 16, (2, 1), 0.5),
    (17, 32, 17, 8, (4, 2), 0.61),          # stride 4
    (33, 64, 17, 64, (3, 3), 0.4),          # coarser latitudes, same longitudes
    (33, 64, 33, 64, (1,), 0.3),
    (25, 48, 25, 48, (5, 4), 1.1),
    (33, 64, 33, 64, (3, 3), 3.0),          # cap covering almost the whole sphere
])
def test_builder_matches_oracle_small(case):
    lib, ref = _pair(*case)
    _compare(lib, ref)


def test_default_cutoff():
    lib = sdc.psi_build(33, 64, 33, 64, (3,), None)
    assert lib.theta_cutoff == pytest.approx(4 * math.pi / 32, rel=1e-15)
    lib2 = sdc.psi_build(721, 1440, 361, 720, (5, 4), None)
    assert lib2.theta_cutoff == pytest.approx(6 * math.pi / 360, rel=1e-15)


def test_int_kernel_shape_is_isotropic():
    a = sdc.psi_build(33, 64, 33, 64, 3, 0.4)
    b = sdc.psi_build(33, 64, 33, 64, (3,), 0.4)
    assert a.K == b.K == 3
    for u, v in zip(a.export(), b.export()):
        assert np.array_equal(u, v)


def test_builder_deterministic():
    a = sdc.psi_build(129, 256, 129, 256, (3, 3), 4 * math.pi / 128)
    b = sdc.psi_build(129, 256, 129, 256, (3, 3), 4 * math.pi / 128)
    for u, v in zip(a.export(), b.export()):
        assert np.array_equal(u, v)


def test_query_counts():
    wl = WORKLOADS["c4"]
    p = sdc.psi_build(wl.nlat_in, wl.nlon_in, wl.nlat_out, wl.nlon_out, wl.kernel_shape,
                      wl.theta_cutoff)
    assert (p.K, p.nnz, p.nnz_nonzero) == (7, 156997, 555973)


# the other latitude grids (DistributedSpectralConvS2 page, grid_in / grid_out):
# the builder computes its nodes and weights by its own Newton iterations, the
# oracle by numpy's Gauss routine and closed forms
GRID_CASES = [
    ("legendre-gauss", "legendre-gauss", (32, 64, 32, 64, (3, 3), 0.45)),
    ("lobatto", "lobatto", (33, 64, 33, 64, (3,), 0.5)),
    ("equiangular-trapezoidal", "equiangular-trapezoidal", (33, 64, 33, 64, (2, 2), 0.4)),
    ("legendre-gauss", "equiangular", (48, 96, 25, 48, (3, 3), 0.5)),   # stride 2
    ("equiangular", "lobatto", (33, 64, 17, 64, (4,), 0.6)),
    ("lobatto", "legendre-gauss", (21, 40, 20, 40, (3, 3), 3.0)),        # nearly whole sphere
    ("legendre-gauss", "legendre-gauss", (1 + 64, 128, 64, 128, (5, 4), 0.3)),
]


@pytest.mark.parametrize("gin,gout,case", GRID_CASES,
                         ids=[f"{a}-{b}-{c[0]}" for a, b, c in GRID_CASES])
def test_builder_matches_oracle_other_grids(gin, gout, case):
    nli, nfi, nlo, nfo, ks, cut = case
    lib = sdc.psi_build(nli, nfi, nlo, nfo, ks, cut, grid_in=gin, grid_out=gout)
    ref = oracle.psi(oracle.Desc(nli, nfi, nlo, nfo, tuple(ks), cut, grid_in=gin, grid_out=gout))
    _compare(lib, ref)


def test_unknown_grid_is_rejected():
    with pytest.raises(NotImplementedError):
        sdc.psi_build(9, 16, 9, 16, (3,), 0.5, grid_in="healpix")
