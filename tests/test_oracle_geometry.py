"""Pins of the oracle's geometry, support rule and index mapping.

P5 compares the oracle (CSR rows, p-shift, rotation) with a brute-force dense
quadrature that loops over every pair of output and input grid points and
uses independent formulas: haversine distance, forward bearing, and weights
from Chebyshev moment equations.  P7 pins the azimuth convention with a closed
form for a linear field.  P8 checks the symmetries of Psi.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import Desc


# ---------------------------------------------------------------------------
# brute force (independent of the oracle's code)
# ---------------------------------------------------------------------------
def _cc_weights_by_moments(nlat):
    n = nlat - 1
    x = np.cos(np.pi * np.arange(nlat) / n)
    T = np.cos(np.outer(np.arange(nlat), np.pi * np.arange(nlat) / n))
    mom = np.array([2.0 / (1.0 - m * m) if m % 2 == 0 else 0.0 for m in range(nlat)])
    return np.linalg.solve(T, mom), x


def _hat(u, c, h):
    return np.maximum(0.0, 1.0 - np.abs(u - c) / h)


def _basis_bf(kernel_shape, cutoff, r, alpha):
    nr = kernel_shape[0]
    if nr == 1:
        rad = [np.ones_like(r)]
    else:
        h = cutoff / (nr - 1)
        rad = [_hat(r, n * h, h) for n in range(nr)]
    if len(kernel_shape) == 1:
        return rad
    nphi = kernel_shape[1]
    out = [rad[0]]
    for n in range(1, nr):
        for m in range(nphi):
            if nphi == 1:
                az = np.ones_like(alpha)
            else:
                wdt = 2 * math.pi / nphi
                d = np.abs((alpha - m * wdt + math.pi) % (2 * math.pi) - math.pi)
                az = np.maximum(0.0, 1.0 - d / wdt)
            out.append(rad[n] * az)
    return out


def brute_force_forward(nlat_in, nlon_in, nlat_out, nlon_out, kernel_shape, cutoff,
                        x, w, groups):
    """Dense spherical quadrature of the compact-support convolution, pair by
    pair, with haversine distance and forward bearing (alpha = pi - bearing)."""
    wcc, _ = _cc_weights_by_moments(nlat_in)
    om = wcc * 2 * math.pi / nlon_in
    lat_in = math.pi / 2 - np.pi * np.arange(nlat_in) / (nlat_in - 1)
    lat_out = math.pi / 2 - np.pi * np.arange(nlat_out) / (nlat_out - 1)
    lon_in = 2 * np.pi * np.arange(nlon_in) / nlon_in
    lon_out = 2 * np.pi * np.arange(nlon_out) / nlon_out
    # all pairs: outputs (j, q) x inputs (i, P)
    L1 = lat_out[:, None, None, None]
    L2 = lat_in[None, None, :, None]
    dl = lon_in[None, None, None, :] - lon_out[None, :, None, None]
    hav = np.sin((L2 - L1) / 2) ** 2 + np.cos(L1) * np.cos(L2) * np.sin(dl / 2) ** 2
    hav = np.clip(hav, 0.0, 1.0)
    r = 2 * np.arctan2(np.sqrt(hav), np.sqrt(1 - hav))
    bearing = np.arctan2(np.sin(dl) * np.cos(L2),
                         np.cos(L1) * np.sin(L2) - np.sin(L1) * np.cos(L2) * np.cos(dl))
    alpha = (math.pi - bearing) % (2 * math.pi)
    inside = r < cutoff * (1 - 1e-10)
    basis = _basis_bf(kernel_shape, cutoff, r, alpha)
    K = len(basis)
    B, Ci = x.shape[:2]
    # X_K[b, ci, k, j, q] = sum_{i,P} basis_k * om_i * x[b, ci, i, P] over the cap
    xk = np.zeros((B, Ci, K, nlat_out, nlon_out))
    for k in range(K):
        Wk = np.where(inside, basis[k], 0.0) * om[None, None, :, None]
        xk[:, :, k] = np.einsum("jqip,bcip->bcjq", Wk, x)
    Co = w.shape[0]
    cig, cog = Ci // groups, Co // groups
    g = np.zeros((B, Co, nlat_out, nlon_out))
    for gr in range(groups):
        g[:, gr * cog:(gr + 1) * cog] = np.einsum(
            "oik,bikjq->bojq", w[gr * cog:(gr + 1) * cog], xk[:, gr * cig:(gr + 1) * cig])
    return xk, g


BF_CASES = [
    # (nlat_in, nlon_in, nlat_out, nlon_out, kernel_shape, cutoff, groups, Ci, Co)
    (9, 16, 9, 16, (3,), 3 * math.pi / 8, 1, 2, 3),
    (17, 32, 17, 32, (3, 3), 4 * math.pi / 16 + 0.013, 1, 3, 2),
    (17, 32, 9, 16, (3, 3), 3 * math.pi / 8 * 0.77, 1, 2, 2),      # stride 2
    (33, 64, 33, 64, (3, 3), 4 * math.pi / 32, 1, 2, 4),           # cutoff on the lattice
    (33, 64, 17, 16, (5, 4), 6 * math.pi / 16 * 0.61, 2, 4, 2),    # stride 4, groups
    (17, 32, 17, 32, (1,), 0.5, 1, 1, 1),
    (17, 32, 17, 32, (2, 1), 0.45, 1, 2, 2),
    (9, 16, 9, 16, (4, 2), 0.9, 1, 1, 1),
]


@pytest.mark.parametrize("case", BF_CASES)
def test_brute_force_matches_oracle(case):
    nli, nfi, nlo, nfo, ks, cut, groups, Ci, Co = case
    rng = np.random.default_rng(7)
    K = oracle.num_basis(ks)
    x = rng.standard_normal((2, Ci, nli, nfi))
    w = rng.standard_normal((Co, Ci // groups, K))
    xk_bf, g_bf = brute_force_forward(nli, nfi, nlo, nfo, ks, cut, x, w, groups)
    d = Desc(nli, nfi, nlo, nfo, ks, cut)
    xk = oracle.contract(d, x)
    g = oracle.einsum(xk, w, groups)
    assert np.linalg.norm(xk - xk_bf) <= 1e-12 * np.linalg.norm(xk_bf)
    assert np.linalg.norm(g - g_bf) <= 1e-12 * np.linalg.norm(g_bf)
    # and element-wise
    assert np.max(np.abs(g - g_bf)) <= 1e-11 * np.max(np.abs(g_bf))


def test_rotation_matches_haversine_and_bearing():
    # r and alpha from the oracle's rotation against haversine and bearing on
    # random points, including output points close to both poles.
    rng = np.random.default_rng(3)
    for th_o in [1e-6, 0.3, 1.2, math.pi / 2, 2.9, math.pi - 1e-6]:
        th = rng.uniform(0, math.pi, 400)
        lam = rng.uniform(0, 2 * math.pi, 400)
        r, a = oracle.rotated_coordinates(th_o, th, lam)
        L1, L2 = math.pi / 2 - th_o, math.pi / 2 - th
        hav = np.sin((L2 - L1) / 2) ** 2 + math.cos(L1) * np.cos(L2) * np.sin(lam / 2) ** 2
        r_h = 2 * np.arctan2(np.sqrt(hav), np.sqrt(1 - hav))
        b = np.arctan2(np.sin(lam) * np.cos(L2),
                       math.cos(L1) * np.sin(L2) - math.sin(L1) * np.cos(L2) * np.cos(lam))
        a_h = (math.pi - b) % (2 * math.pi)
        assert np.max(np.abs(r - r_h)) < 1e-12
        da = np.abs((a - a_h + math.pi) % (2 * math.pi) - math.pi)
        far = r > 1e-6
        assert np.max(da[far]) < 1e-9


# ---------------------------------------------------------------------------
# P7: linear field, anisotropic basis: pins the azimuth zero and direction
# ---------------------------------------------------------------------------
def _gl_integral(f, a, b, n=40):
    t, wt = np.polynomial.legendre.leggauss(n)
    u = 0.5 * (b - a) * t + 0.5 * (b + a)
    return 0.5 * (b - a) * np.sum(wt * f(u))


def _radial_moments(nr, cutoff, n):
    """int phi_n(r) cos r sin r dr and int phi_n(r) sin^2 r dr over [0, cutoff],
    by Gauss-Legendre on each linear piece."""
    h = cutoff / (nr - 1)
    lo, hi = max(0.0, (n - 1) * h), min(cutoff, (n + 1) * h)
    phi = lambda u: np.maximum(0.0, 1.0 - np.abs(u - n * h) / h)
    pieces = [(lo, n * h), (n * h, hi)]
    m1 = sum(_gl_integral(lambda u: phi(u) * np.cos(u) * np.sin(u), a, b) for a, b in pieces if b > a)
    m2 = sum(_gl_integral(lambda u: phi(u) * np.sin(u) ** 2, a, b) for a, b in pieces if b > a)
    return m1, m2


def _linear_field_closed_form(kernel_shape, cutoff, th0, lam0, a_vec, flip=None):
    nr, nphi = kernel_shape
    x0 = np.array([math.sin(th0) * math.cos(lam0), math.sin(th0) * math.sin(lam0), math.cos(th0)])
    e1 = np.array([math.cos(th0) * math.cos(lam0), math.cos(th0) * math.sin(lam0), -math.sin(th0)])
    e2 = np.array([-math.sin(lam0), math.cos(lam0), 0.0])
    if flip == "mirror":
        e2 = -e2
    elif flip == "rot90":
        e1, e2 = e2, -e1
    width = 2 * math.pi / nphi
    out = []
    m1, _ = _radial_moments(nr, cutoff, 0)
    out.append(a_vec @ x0 * 2 * math.pi * m1)
    for n in range(1, nr):
        m1, m2 = _radial_moments(nr, cutoff, n)
        for m in range(nphi):
            am = m * width
            out.append(a_vec @ x0 * width * m1
                       + m2 * 2 * (1 - math.cos(width)) / width
                       * (math.cos(am) * (a_vec @ e1) + math.sin(am) * (a_vec @ e2)))
    return np.array(out)


@pytest.mark.parametrize("kernel_shape", [(3, 3), (3, 4), (2, 5)])
def test_linear_field_anisotropic(kernel_shape):
    cutoff = 0.5 + 0.0037        # off the lattice
    a_vec = np.array([0.3, -0.7, 0.55])
    errs = []
    for nlat in (181, 361):
        nlon = 2 * (nlat - 1)
        d = Desc(nlat, nlon, nlat, nlon, kernel_shape, cutoff)
        th = oracle.colatitudes(nlat)
        lam = oracle.longitudes(nlon)
        f = (a_vec[0] * np.sin(th)[:, None] * np.cos(lam)[None, :]
             + a_vec[1] * np.sin(th)[:, None] * np.sin(lam)[None, :]
             + a_vec[2] * np.cos(th)[:, None])
        j = int(round(0.9 / math.pi * (nlat - 1)))
        q = nlon // 7
        xk = oracle.contract_row(d, f[None, None], oracle.psi_row(d, j))[0, 0, :, q]
        exact = _linear_field_closed_form(kernel_shape, cutoff, th[j], 2 * math.pi * q / nlon, a_vec)
        scale = np.max(np.abs(exact))
        errs.append(np.max(np.abs(xk - exact)) / scale)
        # a mirrored or rotated azimuth convention is off by O(1)
        for flip in ("mirror", "rot90"):
            wrong = _linear_field_closed_form(kernel_shape, cutoff, th[j], 2 * math.pi * q / nlon,
                                              a_vec, flip)
            assert np.max(np.abs(xk - wrong)) / scale > 0.05
    assert errs[1] < 2e-2, errs
    assert errs[1] < errs[0], errs       # converges under refinement


# ---------------------------------------------------------------------------
# P8: symmetries of Psi
# ---------------------------------------------------------------------------
def _as_dense(csr, d, j):
    a, b = int(csr.row_ptr[j]), int(csr.row_ptr[j + 1])
    dense = np.zeros((d.K, d.nlat_in, d.nlon_in))
    dense[:, csr.in_lat[a:b], csr.lon_off[a:b]] = csr.vals[a:b].T
    return dense


def _k_index(n, m, nphi):
    return 1 + (n - 1) * nphi + m


@pytest.mark.parametrize("kernel_shape", [(3,), (3, 3), (3, 4), (5, 4)])
def test_longitude_reflection(kernel_shape):
    d = Desc(33, 64, 33, 64, kernel_shape, 4.4 * math.pi / 32)
    csr = oracle.psi(d)
    nr = kernel_shape[0]
    nphi = kernel_shape[1] if len(kernel_shape) > 1 else 0
    perm = list(range(d.K))
    if nphi:
        for n in range(1, nr):
            for m in range(nphi):
                perm[_k_index(n, m, nphi)] = _k_index(n, (-m) % nphi, nphi)
    pneg = (-np.arange(d.nlon_in)) % d.nlon_in
    for j in range(d.nlat_out):
        D = _as_dense(csr, d, j)
        R = D[perm][:, :, pneg]
        assert np.max(np.abs(D - R)) < 1e-13 * max(1.0, np.max(np.abs(D)))


@pytest.mark.parametrize("kernel_shape", [(3,), (3, 4), (5, 4), (2, 2)])
def test_hemisphere_flip(kernel_shape):
    d = Desc(33, 64, 33, 64, kernel_shape, 4.4 * math.pi / 32)
    csr = oracle.psi(d)
    nr = kernel_shape[0]
    nphi = kernel_shape[1] if len(kernel_shape) > 1 else 0
    perm = list(range(d.K))
    if nphi:
        for n in range(1, nr):
            for m in range(nphi):
                perm[_k_index(n, m, nphi)] = _k_index(n, (nphi // 2 - m) % nphi, nphi)
    J = d.nlat_out - 1
    for j in range(d.nlat_out):
        D = _as_dense(csr, d, j)
        F = _as_dense(csr, d, J - j)[:, ::-1, :]
        assert np.max(np.abs(D[perm] - F)) < 1e-13 * max(1.0, np.max(np.abs(D))), j


def test_isotropic_pole_row_constant_in_longitude():
    d = Desc(33, 64, 33, 64, (3,), 4 * math.pi / 32)
    csr = oracle.psi(d)
    for j in (0, d.nlat_out - 1):
        D = _as_dense(csr, d, j)
        assert np.max(np.abs(D - D[:, :, :1])) < 1e-15


def test_support_windows_are_contiguous_and_symmetric():
    # the cap meets every latitude circle in one longitude interval centred
    # on the output longitude: offsets are {-P..P} mod nlon or the full ring
    for key in ("c1", "c2", "c3"):
        from disco_workloads import WORKLOADS
        wl = WORKLOADS[key]
        d = Desc(wl.nlat_in, wl.nlon_in, wl.nlat_out, wl.nlon_out, wl.kernel_shape, wl.theta_cutoff)
        csr = oracle.psi(d)
        for j in range(0, d.nlat_out, 7):
            a, b = int(csr.row_ptr[j]), int(csr.row_ptr[j + 1])
            for i in np.unique(csr.in_lat[a:b]):
                p = np.sort(csr.lon_off[a:b][csr.in_lat[a:b] == i])
                if p.size == d.nlon_in:
                    continue
                P = (p.size - 1) // 2
                assert p.size == 2 * P + 1
                expect = np.sort(np.arange(-P, P + 1) % d.nlon_in)
                assert np.array_equal(p, expect)
