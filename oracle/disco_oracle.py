"""Plain CPU oracle of the forward DISCO convolution on the 2-sphere, and of
its gradients (the adjoints of its two linear maps, at the end of the file).

TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
C-ABI library and its Python binding) never calls it, and it imports nothing
from the product.  It is slow on purpose: every step is the definition written
out in float64, in the order the pages state it, so that a reader can check it
by eye.

What it computes (torch_harmonics.DiscreteContinuousConvS2 page, forward
equation and the paragraph after it):

    g[b, co, j, q] = sum_{ci, k} w[co, ci, k]
                     * sum_{(i, p)} Psi[k, j, (i, p)] * f[b, ci, i, (q*s + p) mod nlon_in]

with s = nlon_in / nlon_out.  Psi holds the filter-basis values at the input
grid points seen from the output point (theta'_j, 0) after rotating that point
to the north pole, times the quadrature weights; it does not depend on the
output longitude (the p-shift symmetry stated on the same page).

Points the pages leave open, and the reading taken here:

* grid: equiangular colatitudes theta_i = pi*i/(nlat-1), both poles included;
  longitudes lambda_p = 2*pi*p/nlon;
* quadrature: Clenshaw-Curtis weights in cos(theta) times 2*pi/nlon_in;
* the other latitude grids the pages name for grid_in / grid_out (the
  DistributedSpectralConvS2 page lists "legendre-gauss", "lobatto" and
  "equiangular-trapezoidal" beside "equiangular") are read as rules in
  x = cos(theta) over [-1, 1]: Gauss-Legendre nodes and weights;
  Gauss-Lobatto-Legendre nodes (both poles) and weights; equiangular nodes
  with the composite trapezoid rule in x.  The default theta_cutoff formula
  is the same for every grid;
* rotation: about the y axis by -theta'_j, so (theta'_j, 0) goes to the pole;
  r is the polar angle after the rotation, alpha its azimuth, alpha = 0 points
  to local south (+theta) and alpha = pi/2 to local east (+lambda);
* support: r < theta_cutoff * (1 - 1e-10); points at r = theta_cutoff are out;
* basis (piecewise linear): radial hats phi_n(r) = max(0, 1 - |r - n*D|/D),
  D = theta_cutoff/(nr-1); nr = 1 is the cap indicator.  Isotropic
  kernel_shape (nr,) has K = nr.  Anisotropic (nr, nphi) has
  K = 1 + (nr-1)*nphi: phi_0, then phi_n * psi_m, radial index major, with
  periodic azimuthal hats psi_m(alpha) of width 2*pi/nphi centred at
  2*pi*m/nphi; nphi = 1 means psi = 1;
* no basis normalisation, no bias;
* default theta_cutoff (when None): (nr+1)*pi/(nlat_out-1);
* weight layout [Co, Ci/groups, K].

Parity pins for every function live in tests/test_oracle_*.py.
"""
from __future__ import annotations

import functools
import math
from dataclasses import dataclass

import numpy as np

TIE_REL = 1e-10


# --------------------------------------------------------------------------
# Problem description
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Desc:
    """Shapes and basis of one DISCO layer (same fields as the layer's
    constructor on the DiscreteContinuousConvS2 page: in_shape, out_shape,
    kernel_shape, theta_cutoff, grid_in, grid_out)."""
    nlat_in: int
    nlon_in: int
    nlat_out: int
    nlon_out: int
    kernel_shape: tuple
    theta_cutoff: float | None = None
    grid_in: str = "equiangular"
    grid_out: str = "equiangular"

    @property
    def nr(self) -> int:
        return int(self.kernel_shape[0])

    @property
    def nphi(self) -> int:
        return int(self.kernel_shape[1]) if len(self.kernel_shape) > 1 else 0

    @property
    def K(self) -> int:
        return num_basis(self.kernel_shape)

    @property
    def stride(self) -> int:
        return self.nlon_in // self.nlon_out

    @property
    def cutoff(self) -> float:
        if self.theta_cutoff is None:
            return (self.nr + 1) * math.pi / (self.nlat_out - 1)
        return float(self.theta_cutoff)


def num_basis(kernel_shape) -> int:
    """Number of basis functions K for a piecewise-linear kernel_shape."""
    nr = int(kernel_shape[0])
    if len(kernel_shape) == 1:
        return nr
    nphi = int(kernel_shape[1])
    return 1 + (nr - 1) * nphi


# --------------------------------------------------------------------------
# Grid and quadrature
# --------------------------------------------------------------------------
GRIDS = ("equiangular", "legendre-gauss", "lobatto", "equiangular-trapezoidal")


def colatitudes(nlat: int, grid: str = "equiangular") -> np.ndarray:
    """Colatitudes of a latitude grid, ascending from the north pole."""
    if grid in ("equiangular", "equiangular-trapezoidal"):
        return np.array([math.pi * i / (nlat - 1) for i in range(nlat)], dtype=np.float64)
    return np.arccos(grid_rule(nlat, grid)[0])


def grid_rule(nlat: int, grid: str):
    """Nodes x_i = cos(theta_i) (descending, so theta ascends) and weights w_i
    of the grid's rule for int_{-1}^{1} f(x) dx (fresh copies)."""
    x, w = _grid_rule_cached(int(nlat), grid)
    return x.copy(), w.copy()


@functools.lru_cache(maxsize=32)
def _grid_rule_cached(nlat: int, grid: str):
    if grid == "equiangular":
        return np.cos(colatitudes(nlat)), clenshaw_curtis_weights(nlat)
    if grid == "legendre-gauss":
        # Gauss-Legendre: the roots of P_nlat and their Christoffel weights
        # (numpy's Golub-Welsch routine as a library step), nodes descending
        x, w = np.polynomial.legendre.leggauss(nlat)
        return x[::-1].copy(), w[::-1].copy()
    if grid == "lobatto":
        # Gauss-Lobatto-Legendre with n = nlat nodes: x = +-1 and the n - 2
        # roots of P'_{n-1}, which are the roots of the (1, 1) Jacobi
        # polynomial of degree n - 2: the eigenvalues of its symmetric Jacobi
        # matrix (zero diagonal, off-diagonal sqrt(k (k+2) / ((2k+1)(2k+3))),
        # k = 1 .. n-3); w_i = 2 / (n (n-1) P_{n-1}(x_i)^2)
        n = nlat
        if n < 2:
            raise ValueError("a Lobatto grid needs at least 2 nodes")
        m = n - 2
        if m > 0:
            k = np.arange(1, m, dtype=np.float64)
            off = np.sqrt(k * (k + 2.0) / ((2.0 * k + 1.0) * (2.0 * k + 3.0)))
            jac = np.diag(off, 1) + np.diag(off, -1)
            inner = np.sort(np.linalg.eigvalsh(jac))[::-1]
        else:
            inner = np.zeros(0)
        x = np.concatenate([[1.0], inner, [-1.0]])
        pn1 = np.polynomial.legendre.legval(x, np.eye(n)[n - 1])
        w = 2.0 / (n * (n - 1) * pn1 ** 2)
        return x, w
    if grid == "equiangular-trapezoidal":
        # composite trapezoid rule in x on the equiangular nodes:
        # w_i = (x_{i-1} - x_{i+1}) / 2, halves at the two ends
        x = np.cos(colatitudes(nlat))
        w = np.zeros(nlat, dtype=np.float64)
        for i in range(nlat - 1):
            h = x[i] - x[i + 1]
            w[i] += 0.5 * h
            w[i + 1] += 0.5 * h
        return x, w
    raise ValueError(f"unknown grid {grid!r} (known: {GRIDS})")


def longitudes(nlon: int) -> np.ndarray:
    """Equispaced longitudes 2*pi*p/nlon."""
    return np.array([2.0 * math.pi * p / nlon for p in range(nlon)], dtype=np.float64)


def clenshaw_curtis_weights(nlat: int) -> np.ndarray:
    """Clenshaw-Curtis weights for nodes cos(theta_i), integrating over [-1, 1].

    Closed form of Clenshaw and Curtis (1960): with n = nlat - 1,
    w_i = (c_i/n) * (1 - sum_{k=1}^{n//2} b_k/(4k^2-1) * cos(2k theta_i)),
    c_0 = c_n = 1, c_i = 2 otherwise, b_k = 1 if 2k = n else 2.
    """
    n = nlat - 1
    theta = colatitudes(nlat)
    w = np.zeros(nlat, dtype=np.float64)
    for i in range(nlat):
        acc = 0.0
        for k in range(1, n // 2 + 1):
            b = 1.0 if 2 * k == n else 2.0
            acc += b / (4.0 * k * k - 1.0) * math.cos(2.0 * k * theta[i])
        c = 1.0 if i in (0, n) else 2.0
        w[i] = c / n * (1.0 - acc)
    return w


def quadrature_weights(nlat: int, nlon: int, grid: str = "equiangular") -> np.ndarray:
    """Per-point spherical quadrature weight of latitude row i (sums to 4*pi
    over the whole grid): the grid's rule in cos(theta) (Clenshaw-Curtis for
    the equiangular grid) times 2*pi/nlon."""
    return grid_rule(nlat, grid)[1] * (2.0 * math.pi / nlon)


# --------------------------------------------------------------------------
# Geometry: input points seen from an output point rotated to the pole
# --------------------------------------------------------------------------
def rotated_coordinates(theta_out: float, theta_in: np.ndarray, lam: np.ndarray):
    """Polar angle r and azimuth alpha of input points (theta_in, lam) after
    the rotation that takes the output point (theta_out, 0) to the north pole.

    The rotation is about the y axis by -theta_out.  alpha = 0 is local south
    (+theta), alpha = pi/2 local east (+lambda).  Returns arrays shaped like
    the broadcast of theta_in and lam.
    """
    theta_in, lam = np.broadcast_arrays(np.asarray(theta_in, np.float64),
                                        np.asarray(lam, np.float64))
    x = np.sin(theta_in) * np.cos(lam)
    y = np.sin(theta_in) * np.sin(lam)
    z = np.cos(theta_in)
    ct, st = math.cos(theta_out), math.sin(theta_out)
    xr = x * ct - z * st
    yr = y
    zr = x * st + z * ct
    r = np.arctan2(np.sqrt(xr * xr + yr * yr), zr)
    alpha = np.mod(np.arctan2(yr, xr), 2.0 * math.pi)
    return r, alpha


# --------------------------------------------------------------------------
# Piecewise-linear filter basis
# --------------------------------------------------------------------------
def radial_hat(n: int, nr: int, cutoff: float, r: np.ndarray) -> np.ndarray:
    """phi_n(r): hat of half-width D = cutoff/(nr-1) centred at n*D.
    For nr = 1 the single radial function is the cap indicator (value 1)."""
    if nr == 1:
        return np.ones_like(r)
    d = cutoff / (nr - 1)
    return np.maximum(0.0, 1.0 - np.abs(r - n * d) / d)


def azimuthal_hat(m: int, nphi: int, alpha: np.ndarray) -> np.ndarray:
    """psi_m(alpha): periodic hat of half-width 2*pi/nphi centred at
    2*pi*m/nphi (circular distance); identically 1 when nphi = 1."""
    if nphi == 1:
        return np.ones_like(alpha)
    width = 2.0 * math.pi / nphi
    diff = np.mod(alpha - m * width, 2.0 * math.pi)
    dist = np.minimum(diff, 2.0 * math.pi - diff)
    return np.maximum(0.0, 1.0 - dist / width)


def basis_values(kernel_shape, cutoff: float, r: np.ndarray, alpha: np.ndarray) -> np.ndarray:
    """All K basis functions at the points (r, alpha); shape [K, npoints]."""
    nr = int(kernel_shape[0])
    r = np.asarray(r, np.float64)
    alpha = np.asarray(alpha, np.float64)
    if len(kernel_shape) == 1:
        return np.stack([radial_hat(n, nr, cutoff, r) for n in range(nr)])
    nphi = int(kernel_shape[1])
    rows = [radial_hat(0, nr, cutoff, r)]
    for n in range(1, nr):
        for m in range(nphi):
            rows.append(radial_hat(n, nr, cutoff, r) * azimuthal_hat(m, nphi, alpha))
    return np.stack(rows)


# --------------------------------------------------------------------------
# Psi: the sparse convolution tensor, canonical per-output-row CSR
# --------------------------------------------------------------------------
@dataclass
class PsiCSR:
    """Psi[k, j, (i, p)] as CSR over output rows j.

    row_ptr [nlat_out+1] int64; in_lat, lon_off [nnz] int32 (input row i and
    longitude offset p of each support point, sorted by (i, p)); vals [nnz, K]
    float64 (all K values per support point, zeros kept).
    """
    row_ptr: np.ndarray
    in_lat: np.ndarray
    lon_off: np.ndarray
    vals: np.ndarray

    @property
    def nnz(self) -> int:
        return int(self.row_ptr[-1])


def psi_row(desc: Desc, j: int, omega: np.ndarray | None = None):
    """Support points and values of output row j: (in_lat, lon_off, vals).
    `omega` may pass in quadrature_weights(nlat_in, nlon_in) to save time."""
    cutoff = desc.cutoff
    theta_in = colatitudes(desc.nlat_in, desc.grid_in)
    theta_out = colatitudes(desc.nlat_out, desc.grid_out)[j]
    lam = longitudes(desc.nlon_in)
    if omega is None:
        omega = quadrature_weights(desc.nlat_in, desc.nlon_in, desc.grid_in)
    lat_list, lon_list, val_list = [], [], []
    for i in range(desc.nlat_in):
        # r >= |theta_i - theta'_j|, so rows farther away cannot be in the cap
        if abs(theta_in[i] - theta_out) > cutoff:
            continue
        r, alpha = rotated_coordinates(theta_out, np.full(desc.nlon_in, theta_in[i]), lam)
        inside = r < cutoff * (1.0 - TIE_REL)
        p = np.nonzero(inside)[0]
        if p.size == 0:
            continue
        vals = basis_values(desc.kernel_shape, cutoff, r[p], alpha[p]).T * omega[i]
        lat_list.append(np.full(p.size, i, dtype=np.int32))
        lon_list.append(p.astype(np.int32))
        val_list.append(vals)
    if not lat_list:
        return (np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros((0, desc.K)))
    return (np.concatenate(lat_list), np.concatenate(lon_list), np.concatenate(val_list))


def psi(desc: Desc) -> PsiCSR:
    """The whole Psi tensor as canonical CSR (sorted by j, then i, then p)."""
    row_ptr = np.zeros(desc.nlat_out + 1, dtype=np.int64)
    omega = quadrature_weights(desc.nlat_in, desc.nlon_in, desc.grid_in)
    lats, lons, vals = [], [], []
    for j in range(desc.nlat_out):
        a, b, v = psi_row(desc, j, omega)
        lats.append(a)
        lons.append(b)
        vals.append(v)
        row_ptr[j + 1] = row_ptr[j] + a.size
    return PsiCSR(row_ptr, np.concatenate(lats).astype(np.int32),
                  np.concatenate(lons).astype(np.int32),
                  np.concatenate(vals).reshape(-1, desc.K))


# --------------------------------------------------------------------------
# The two sums of the forward equation
# --------------------------------------------------------------------------
def contract_row(desc: Desc, x: np.ndarray, row, cols_out=None) -> np.ndarray:
    """Inner sum of the forward equation for one output row j:
    X_K[b, ci, k, q] = sum_{(i,p) in row j} Psi[k, j, (i,p)] * x[b, ci, i, (q*s+p) mod nlon_in].

    `row` is (in_lat, lon_off, vals) from psi_row; x is [B, Ci, nlat_in, nlon_in].
    `cols_out` optionally restricts q to a list of output longitudes (default:
    all).  Accumulates support points one at a time in canonical order, so
    every output longitude sees the same summation order.
    """
    in_lat, lon_off, vals = row
    x = np.asarray(x, dtype=np.float64)
    B, C = x.shape[:2]
    q = np.arange(desc.nlon_out) if cols_out is None else np.asarray(cols_out, dtype=np.int64)
    out = np.zeros((B, C, desc.K, q.size), dtype=np.float64)
    for e in range(in_lat.size):
        cols = (q * desc.stride + int(lon_off[e])) % desc.nlon_in
        xs = x[:, :, int(in_lat[e]), :][:, :, cols]                # [B, C, len(q)]
        out += vals[e][None, None, :, None] * xs[:, :, None, :]
    return out


def contract(desc: Desc, x: np.ndarray, csr: PsiCSR | None = None, rows=None,
             cols_out=None) -> np.ndarray:
    """X_K[b, ci, k, j, q] for the output rows `rows` (default: all rows) and
    output longitudes `cols_out` (default: all).
    Shape [B, Ci, K, len(rows), len(cols_out)]."""
    if rows is None:
        rows = range(desc.nlat_out)
    rows = list(rows)
    nq = desc.nlon_out if cols_out is None else len(cols_out)
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros((x.shape[0], x.shape[1], desc.K, len(rows), nq))
    omega = None if csr is not None else quadrature_weights(desc.nlat_in, desc.nlon_in,
                                                            desc.grid_in)
    for jj, j in enumerate(rows):
        if csr is not None:
            a, b = int(csr.row_ptr[j]), int(csr.row_ptr[j + 1])
            row = (csr.in_lat[a:b], csr.lon_off[a:b], csr.vals[a:b])
        else:
            row = psi_row(desc, j, omega)
        out[:, :, :, jj, :] = contract_row(desc, x, row, cols_out)
    return out


def einsum(xk: np.ndarray, w: np.ndarray, groups: int) -> np.ndarray:
    """Outer sums of the forward equation:
    g[b, co, j, q] = sum_{ci' < Ci/G} sum_k w[co, ci', k] * X_K[b, G(co)*Ci/G + ci', k, j, q],
    G(co) = co // (Co/G).  xk is [B, Ci, K, H, W], w is [Co, Ci/G, K]."""
    xk = np.asarray(xk, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, Ci, K, H, W = xk.shape
    Co = w.shape[0]
    cig, cog = Ci // groups, Co // groups
    g = np.zeros((B, Co, H, W), dtype=np.float64)
    for grp in range(groups):
        xs = xk[:, grp * cig:(grp + 1) * cig]                     # [B, cig, K, H, W]
        ws = w[grp * cog:(grp + 1) * cog]                           # [cog, cig, K]
        g[:, grp * cog:(grp + 1) * cog] = np.einsum("oik,bikhw->bohw", ws, xs)
    return g


def forward(desc: Desc, x: np.ndarray, w: np.ndarray, groups: int = 1,
            csr: PsiCSR | None = None, rows=None, cols_out=None,
            bias: np.ndarray | None = None) -> np.ndarray:
    """The forward DISCO convolution g [B, Co, len(rows), len(cols_out)] in
    float64, for the output rows `rows` and longitudes `cols_out` (default
    all), plus bias[co] when given (the layer's `bias` parameter)."""
    g = einsum(contract(desc, x, csr=csr, rows=rows, cols_out=cols_out), w, groups)
    if bias is not None:
        g = g + np.asarray(bias, dtype=np.float64)[None, :, None, None]
    return g


# --------------------------------------------------------------------------
# Backward: the gradients the layer's autograd returns.  The pages give no
# formulas; they say the layer trains by backpropagation and that its fused
# mode recomputes X_K in backward instead of saving it (DiscreteContinuousConvS2
# page, `fused` parameter).  The forward is linear in x and in w, so each
# gradient is the adjoint of one of its linear maps, written out here from the
# forward equation.
# --------------------------------------------------------------------------
def contract_transpose(desc: Desc, gxk: np.ndarray, csr: PsiCSR | None = None) -> np.ndarray:
    """Adjoint of `contract`: for every support point (i, p) of every output
    row j and every output longitude q,
        gx[b, c, i, (q*s + p) mod nlon_in] += sum_k Psi[k, j, (i, p)] * gxk[b, c, k, j, q].
    gxk is [B, C, K, nlat_out, nlon_out]; returns gx [B, C, nlat_in, nlon_in]."""
    gxk = np.asarray(gxk, dtype=np.float64)
    B, C = gxk.shape[0], gxk.shape[1]
    if csr is None:
        csr = psi(desc)
    gx = np.zeros((B, C, desc.nlat_in, desc.nlon_in), dtype=np.float64)
    q = np.arange(desc.nlon_out)
    for j in range(desc.nlat_out):
        for e in range(int(csr.row_ptr[j]), int(csr.row_ptr[j + 1])):
            i, p = int(csr.in_lat[e]), int(csr.lon_off[e])
            cols = (q * desc.stride + p) % desc.nlon_in     # distinct for distinct q
            gx[:, :, i, cols] += np.einsum("k,bckq->bcq", csr.vals[e], gxk[:, :, :, j, :])
    return gx


def einsum_grad_w(gg: np.ndarray, xk: np.ndarray, groups: int) -> np.ndarray:
    """Adjoint of `einsum` in w:
    gw[co, ci', k] = sum_{b, j, q} gg[b, co, j, q] * X_K[b, G(co)*Ci/G + ci', k, j, q]."""
    gg = np.asarray(gg, dtype=np.float64)
    xk = np.asarray(xk, dtype=np.float64)
    Co, Ci = gg.shape[1], xk.shape[1]
    cig, cog = Ci // groups, Co // groups
    gw = np.zeros((Co, cig, xk.shape[2]), dtype=np.float64)
    for grp in range(groups):
        gw[grp * cog:(grp + 1) * cog] = np.einsum(
            "bohw,bikhw->oik", gg[:, grp * cog:(grp + 1) * cog], xk[:, grp * cig:(grp + 1) * cig])
    return gw


def einsum_grad_xk(gg: np.ndarray, w: np.ndarray, groups: int) -> np.ndarray:
    """Adjoint of `einsum` in X_K:
    gxk[b, G*Ci/G + ci', k, j, q] = sum_{co in group G} w[co, ci', k] * gg[b, co, j, q]."""
    gg = np.asarray(gg, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, Co, H, W = gg.shape
    cig, K = w.shape[1], w.shape[2]
    cog = Co // groups
    gxk = np.zeros((B, cig * groups, K, H, W), dtype=np.float64)
    for grp in range(groups):
        gxk[:, grp * cig:(grp + 1) * cig] = np.einsum(
            "oik,bohw->bikhw", w[grp * cog:(grp + 1) * cog], gg[:, grp * cog:(grp + 1) * cog])
    return gxk


def backward(desc: Desc, x: np.ndarray, w: np.ndarray, gg: np.ndarray, groups: int = 1,
             csr: PsiCSR | None = None):
    """Gradients (gx, gw) of sum(gg * forward(x, w)) with respect to x and w
    (the bias gradient is gg summed over b, j, q).  X_K is recomputed, as the
    fused mode does."""
    if csr is None:
        csr = psi(desc)
    xk = contract(desc, x, csr=csr)
    gw = einsum_grad_w(gg, xk, groups)
    gx = contract_transpose(desc, einsum_grad_xk(gg, w, groups), csr=csr)
    return gx, gw
