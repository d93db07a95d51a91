"""Pins of the oracle's grid and quadrature weights against mathematics.

The pages only say that Psi is weighted by the quadrature weights and that the
grid is equiangular (DiscreteContinuousConvS2 page, Psi paragraph and the
grid_in parameter).  The weights used are Clenshaw-Curtis in cos(theta); they
are pinned here by facts that do not depend on the oracle's own formula.
"""
import math

import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("nlat", [3, 5, 9, 33, 129, 361, 721])
def test_cc_weights_sum_and_symmetry(nlat):
    # P1: the weights integrate 1 over [-1, 1] exactly, are positive and
    # symmetric; the spherical weights sum to the sphere's area 4*pi.
    w = oracle.clenshaw_curtis_weights(nlat)
    assert abs(w.sum() - 2.0) < 1e-13
    assert np.all(w > 0)
    assert np.allclose(w, w[::-1], rtol=0, atol=1e-15)
    nlon = 2 * (nlat - 1)
    om = oracle.quadrature_weights(nlat, nlon)
    assert abs(om.sum() * nlon - 4 * math.pi) < 1e-12


def test_cc_small_cases_textbook():
    # n = 2 is Simpson's rule; n = 4 Clenshaw-Curtis weights are
    # (1, 8, 12, 8, 1)/15 (textbook values).
    assert np.allclose(oracle.clenshaw_curtis_weights(3), [1 / 3, 4 / 3, 1 / 3], atol=1e-15)
    assert np.allclose(oracle.clenshaw_curtis_weights(5),
                       np.array([1, 8, 12, 8, 1]) / 15.0, atol=1e-15)


@pytest.mark.parametrize("nlat", [9, 33, 65, 129])
def test_cc_polynomial_exactness(nlat):
    # P2: sum_i w_i cos^m(theta_i) = int_{-1}^{1} x^m dx for m <= nlat-1.
    w = oracle.clenshaw_curtis_weights(nlat)
    x = np.cos(oracle.colatitudes(nlat))
    for m in range(nlat):
        exact = 2.0 / (m + 1) if m % 2 == 0 else 0.0
        assert abs(np.dot(w, x ** m) - exact) < 1e-12, m


@pytest.mark.parametrize("nlat", [9, 17, 33, 65])
def test_cc_weights_solve_chebyshev_moments(nlat):
    # The interpolatory rule on Chebyshev extreme points is unique: solving
    # the moment equations in the Chebyshev basis (well conditioned) must give
    # the same weights as the closed form.
    n = nlat - 1
    x = np.cos(np.pi * np.arange(nlat) / n)
    T = np.cos(np.outer(np.arange(nlat), np.arccos(np.clip(x, -1, 1))))
    mom = np.array([2.0 / (1.0 - m * m) if m % 2 == 0 else 0.0 for m in range(nlat)])
    w_solve = np.linalg.solve(T, mom)
    assert np.allclose(w_solve, oracle.clenshaw_curtis_weights(nlat), rtol=0, atol=1e-12)


def test_grid_nodes():
    th = oracle.colatitudes(5)
    assert th[0] == 0.0 and abs(th[-1] - math.pi) < 1e-15
    lam = oracle.longitudes(8)
    assert np.allclose(lam, np.arange(8) * math.pi / 4)


# --------------------------------------------------------------------------
# The other latitude grids the pages name for grid_in / grid_out
# (DistributedSpectralConvS2 page: "legendre-gauss", "lobatto",
# "equiangular-trapezoidal").  The pages define none of them; each is read as
# a rule in x = cos(theta) and pinned by what that rule must satisfy.
# --------------------------------------------------------------------------
def _moment(m):
    return 2.0 / (m + 1) if m % 2 == 0 else 0.0


@pytest.mark.parametrize("grid", ["legendre-gauss", "lobatto", "equiangular-trapezoidal"])
@pytest.mark.parametrize("nlat", [2, 3, 4, 7, 16, 33, 64])
def test_grid_rules_basic(grid, nlat):
    # weights integrate 1 exactly, are positive (the trapezoid gives the
    # poles' zero-width ends half a segment), nodes descend in x (colatitude
    # ascends) inside [-1, 1] and the rule is symmetric about the equator
    x, w = oracle.grid_rule(nlat, grid)
    assert x.shape == w.shape == (nlat,)
    assert abs(w.sum() - 2.0) < 1e-13
    assert np.all(w > 0)
    assert np.all(np.diff(x) < 0) and x[0] <= 1.0 and x[-1] >= -1.0
    assert np.allclose(x, -x[::-1], atol=1e-14)
    assert np.allclose(w, w[::-1], rtol=0, atol=1e-14)
    th = oracle.colatitudes(nlat, grid)
    assert np.allclose(np.cos(th), x, atol=1e-14)
    nlon = 8
    assert abs(oracle.quadrature_weights(nlat, nlon, grid).sum() * nlon - 4 * math.pi) < 1e-12


@pytest.mark.parametrize("nlat", [1, 2, 3, 5, 8, 17, 32])
def test_gauss_legendre_degree(nlat):
    # n Gauss points integrate every polynomial of degree <= 2n - 1 exactly,
    # and not x^(2n): a rule of the wrong size or wrong nodes fails one side
    x, w = oracle.grid_rule(nlat, "legendre-gauss")
    for m in range(2 * nlat):
        assert abs(np.dot(w, x ** m) - _moment(m)) < 1e-13, m
    if nlat <= 8:
        # for x^(2n) the rule falls short by the Gauss error term
        # 2^(2n+1) (n!)^4 / ((2n+1) ((2n)!)^2)
        n = nlat
        term = 2.0 ** (2 * n + 1) * math.factorial(n) ** 4 / ((2 * n + 1) * math.factorial(2 * n) ** 2)
        err = _moment(2 * n) - np.dot(w, x ** (2 * n))
        assert abs(err - term) < 1e-12 * max(1.0, term) and term > 1e-9
    assert np.all(np.abs(x) < 1.0)           # no pole in a Gauss grid


@pytest.mark.parametrize("nlat", [3, 4, 6, 9, 17, 33])
def test_lobatto_degree_and_poles(nlat):
    # n Lobatto points: both end points, exact to degree 2n - 3, not beyond
    x, w = oracle.grid_rule(nlat, "lobatto")
    assert x[0] == 1.0 and x[-1] == -1.0
    th = oracle.colatitudes(nlat, "lobatto")
    assert th[0] == 0.0 and abs(th[-1] - math.pi) < 1e-15
    for m in range(2 * nlat - 2):
        assert abs(np.dot(w, x ** m) - _moment(m)) < 1e-13, m
    if nlat <= 6:
        assert abs(np.dot(w, x ** (2 * nlat - 2)) - _moment(2 * nlat - 2)) > 1e-6


def test_small_rules_textbook():
    # closed forms: Gauss n = 2 at +-1/sqrt(3) with weights 1; Lobatto n = 3
    # at 1, 0, -1 with 1/3, 4/3, 1/3 (Simpson) and n = 4 at +-1, +-1/sqrt(5)
    # with 1/6, 5/6; the trapezoid on colatitudes 0, pi/2, pi is 1/2, 1, 1/2
    x, w = oracle.grid_rule(2, "legendre-gauss")
    assert np.allclose(x, [1 / math.sqrt(3), -1 / math.sqrt(3)], atol=1e-15)
    assert np.allclose(w, [1.0, 1.0], atol=1e-15)
    x, w = oracle.grid_rule(3, "lobatto")
    assert np.allclose(x, [1, 0, -1], atol=1e-15) and np.allclose(w, [1 / 3, 4 / 3, 1 / 3], atol=1e-15)
    x, w = oracle.grid_rule(4, "lobatto")
    assert np.allclose(x, [1, 1 / math.sqrt(5), -1 / math.sqrt(5), -1], atol=1e-15)
    assert np.allclose(w, [1 / 6, 5 / 6, 5 / 6, 1 / 6], atol=1e-15)
    x, w = oracle.grid_rule(3, "equiangular-trapezoidal")
    assert np.allclose(x, [1, 0, -1], atol=1e-15) and np.allclose(w, [0.5, 1.0, 0.5], atol=1e-15)


@pytest.mark.parametrize("nlat", [3, 9, 33])
def test_trapezoid_linear_exact_and_error_term(nlat):
    # the trapezoid integrates linear functions exactly; for x^2 each segment
    # [a, b] overshoots by (b - a)^3 / 6, so the total error is that sum
    x, w = oracle.grid_rule(nlat, "equiangular-trapezoidal")
    assert abs(np.dot(w, x)) < 1e-15 and abs(np.dot(w, np.ones(nlat)) - 2.0) < 1e-14
    h = x[:-1] - x[1:]
    assert abs((np.dot(w, x ** 2) - 2.0 / 3.0) - np.sum(h ** 3) / 6.0) < 1e-14


@pytest.mark.parametrize("grid", ["legendre-gauss", "lobatto", "equiangular-trapezoidal"])
@pytest.mark.parametrize("cutoff", [0.3, 1.2, 3.0])
def test_psi_uses_the_grid_rule(grid, cutoff):
    # seen from the north pole (output row 0 of an equiangular output grid)
    # the cap holds exactly the input rows with theta_i < cutoff, all their
    # longitudes; with the cap indicator (kernel_shape (1,)) the row's Psi
    # sums to 2 pi times those rows' rule weights.  A grid whose nodes or
    # weights were not the ones Psi uses fails this.
    nlat = 37
    x, w = oracle.grid_rule(nlat, grid)
    th = np.arccos(np.clip(x, -1, 1))
    d = oracle.Desc(nlat, 24, 9, 24, (1,), cutoff, grid_in=grid, grid_out="equiangular")
    lat, lon, v = oracle.psi_row(d, 0)
    inside = th < cutoff * (1 - oracle.TIE_REL)
    assert sorted(set(lat.tolist())) == np.nonzero(inside)[0].tolist()
    assert lat.size == 24 * int(inside.sum())
    assert abs(v.sum() - 2 * math.pi * w[inside].sum()) < 1e-12


@pytest.mark.parametrize("grid", ["legendre-gauss", "lobatto"])
def test_rules_at_full_size(grid):
    # 721 rows (the 0.25 degree grids): still symmetric, summing to 2 and
    # integrating low-degree polynomials to rounding
    x, w = oracle.grid_rule(721, grid)
    assert abs(w.sum() - 2.0) < 1e-12
    assert np.allclose(x, -x[::-1], atol=1e-13)
    for m in range(0, 41):
        assert abs(np.dot(w, x ** m) - _moment(m)) < 1e-12, m
