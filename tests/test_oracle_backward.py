"""Pins of the oracle's backward (gradients of the forward DISCO convolution).

The pages state no backward formulas, only that the layer trains and that
the fused mode recomputes X_K in backward (DiscreteContinuousConvS2 page,
`fused` parameter).  The forward is linear in x and in w, so its gradients
are adjoints; they are pinned by the adjoint identities, by exact
directional derivatives of the (bilinear) forward, and by brute force: the
Jacobian assembled column by column from unit inputs on a tiny grid.
"""
import math

import numpy as np
import pytest

import oracle


def _desc(nli, nfi, nlo, nfo, ks, cut, gin="equiangular", gout="equiangular"):
    return oracle.Desc(nli, nfi, nlo, nfo, tuple(ks), cut, grid_in=gin, grid_out=gout)


# Isotropic bases, and anisotropic ones with nphi <= 2, are symmetric under
# the longitude reflection p -> -p, so they cannot tell the shift's sign; the
# nphi = 3 cases can (a sign flipped in contract_transpose fails them).
CASES = [
    _desc(9, 16, 9, 16, (3,), 0.9),
    _desc(17, 32, 9, 16, (2, 1), 0.5),                 # stride 2
    _desc(13, 24, 13, 8, (3, 3), 0.8),                 # stride 3, nphi = 3
    _desc(9, 16, 9, 16, (3, 3), 2.9),                  # cap over almost the sphere
    _desc(12, 16, 7, 16, (2, 3), 0.7, "legendre-gauss", "lobatto"),
]


@pytest.mark.parametrize("d", CASES, ids=range(len(CASES)))
def test_contract_transpose_is_the_adjoint(d):
    # <contract(x), y> = <x, contract_transpose(y)> for random x, y
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 3, d.nlat_in, d.nlon_in))
    y = rng.standard_normal((2, 3, d.K, d.nlat_out, d.nlon_out))
    csr = oracle.psi(d)
    lhs = np.sum(oracle.contract(d, x, csr=csr) * y)
    rhs = np.sum(x * oracle.contract_transpose(d, y, csr=csr))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


@pytest.mark.parametrize("groups,Ci,Co", [(1, 4, 6), (2, 4, 6), (4, 4, 4), (2, 2, 6)])
def test_einsum_gradients_are_adjoints(groups, Ci, Co):
    rng = np.random.default_rng(5)
    K, H, W = 3, 4, 5
    xk = rng.standard_normal((2, Ci, K, H, W))
    w = rng.standard_normal((Co, Ci // groups, K))
    gg = rng.standard_normal((2, Co, H, W))
    g = oracle.einsum(xk, w, groups)
    ip = np.sum(g * gg)
    assert abs(ip - np.sum(w * oracle.einsum_grad_w(gg, xk, groups))) <= 1e-12 * abs(ip)
    assert abs(ip - np.sum(xk * oracle.einsum_grad_xk(gg, w, groups))) <= 1e-12 * abs(ip)


@pytest.mark.parametrize("d,groups", [(CASES[0], 1), (CASES[1], 2), (CASES[2], 1), (CASES[4], 1)])
def test_backward_matches_directional_derivatives(d, groups):
    # the forward is bilinear, so f(x + t dx, w) - f(x, w) = t f(dx, w) and
    # f(x, w + t dw) - f(x, w) = t f(x, dw) exactly; the gradients must give
    # <gg, f(dx, w)> = <gx, dx> and <gg, f(x, dw)> = <gw, dw>
    rng = np.random.default_rng(11)
    Ci, Co = 4, 6
    x = rng.standard_normal((1, Ci, d.nlat_in, d.nlon_in))
    w = rng.standard_normal((Co, Ci // groups, d.K))
    gg = rng.standard_normal((1, Co, d.nlat_out, d.nlon_out))
    dx = rng.standard_normal(x.shape)
    dw = rng.standard_normal(w.shape)
    csr = oracle.psi(d)
    gx, gw = oracle.backward(d, x, w, gg, groups, csr=csr)
    a = np.sum(gg * oracle.forward(d, dx, w, groups, csr=csr))
    b = np.sum(gg * oracle.forward(d, x, dw, groups, csr=csr))
    assert abs(a - np.sum(gx * dx)) <= 1e-11 * max(1.0, abs(a))
    assert abs(b - np.sum(gw * dw)) <= 1e-11 * max(1.0, abs(b))


def test_backward_brute_force_jacobian():
    # tiny grid: assemble d g / d x one unit input at a time and contract it
    # with gg by hand; likewise for every weight
    d = _desc(5, 8, 5, 4, (2, 3), 1.1)      # stride 2, nphi = 3
    rng = np.random.default_rng(2)
    Ci, Co = 2, 3
    x = rng.standard_normal((1, Ci, d.nlat_in, d.nlon_in))
    w = rng.standard_normal((Co, Ci, d.K))
    gg = rng.standard_normal((1, Co, d.nlat_out, d.nlon_out))
    csr = oracle.psi(d)
    gx, gw = oracle.backward(d, x, w, gg, 1, csr=csr)
    gx_bf = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        e = np.zeros_like(x)
        e[idx] = 1.0
        gx_bf[idx] = np.sum(gg * oracle.forward(d, e, w, 1, csr=csr))
    gw_bf = np.zeros_like(w)
    for idx in np.ndindex(*w.shape):
        e = np.zeros_like(w)
        e[idx] = 1.0
        gw_bf[idx] = np.sum(gg * oracle.forward(d, x, e, 1, csr=csr))
    assert np.allclose(gx, gx_bf, rtol=1e-12, atol=1e-12)
    assert np.allclose(gw, gw_bf, rtol=1e-12, atol=1e-12)
    assert np.abs(gx).max() > 0 and np.abs(gw).max() > 0
