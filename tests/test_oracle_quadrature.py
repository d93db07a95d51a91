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
