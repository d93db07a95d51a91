// Host-side builder of the DISCO convolution tensor Psi, in float64.
//
// Psi[k, j, (i, p)] is the value of basis function k at input grid point
// (theta_i, lambda_p) as seen from output point (theta'_j, 0) once that point
// is rotated to the north pole, times the quadrature weight of the input point
// (torch_harmonics.DiscreteContinuousConvS2 page, the paragraph after the
// forward equation).  Because longitudes are equispaced, one row of Psi per
// output latitude serves every output longitude (p-shift symmetry, same page).
//
// Conventions where the pages are silent (each is a reading):
//  * equiangular grid with both poles, theta_i = pi*i/(nlat-1);
//  * Clenshaw-Curtis weights in cos(theta), times 2*pi/nlon_in;
//  * the other grids the pages name ("legendre-gauss", "lobatto",
//    "equiangular-trapezoidal", DistributedSpectralConvS2 page) as rules in
//    x = cos(theta) over [-1, 1]: Gauss-Legendre; Gauss-Lobatto-Legendre
//    (both poles); equiangular nodes with the composite trapezoid in x;
//  * local frame at the output point: alpha = 0 towards +theta (south),
//    alpha = pi/2 towards +lambda (east); r is the great-circle distance;
//  * support is r < cutoff*(1 - 1e-10): points at r == cutoff are excluded;
//  * piecewise-linear hats: phi_n(r) = max(0, 1 - |r - n*D|/D), D = cutoff/(nr-1),
//    nr == 1 gives the cap indicator; anisotropic k = 1 + (n-1)*nphi + m carries
//    phi_n(r)*psi_m(alpha), psi_m a periodic hat of width 2*pi/nphi centred at
//    2*pi*m/nphi (psi = 1 when nphi == 1); k = 0 carries phi_0;
//  * no normalisation of the basis.
#include <cmath>
#include <cstdlib>
#include <new>

#include "disco_internal.h"

namespace disco {
namespace {

constexpr double kPi = 3.141592653589793238462643383279502884;
constexpr double kTieRel = 1e-10;
constexpr int kMaxK = 64;

// Clenshaw-Curtis weights on the nodes x_i = cos(pi*i/n), i = 0..n, for the
// integral over [-1, 1].  Written as the cosine series of the interpolating
// polynomial's integral (Clenshaw & Curtis 1960).
std::vector<double> clenshaw_curtis(int nlat) {
    const int n = nlat - 1;
    std::vector<double> w(nlat);
    for (int i = 0; i <= n; ++i) {
        const double th = kPi * double(i) / double(n);
        double s = 0.0;
        for (int k = 1; 2 * k <= n; ++k) {
            const double bk = (2 * k == n) ? 1.0 : 2.0;
            s += bk * std::cos(2.0 * k * th) / (4.0 * double(k) * double(k) - 1.0);
        }
        const double ci = (i == 0 || i == n) ? 1.0 : 2.0;
        w[i] = ci * (1.0 - s) / double(n);
    }
    return w;
}

// Legendre P_m(x) and P_{m-1}(x) by the three-term recurrence
// (k P_k = (2k - 1) x P_{k-1} - (k - 1) P_{k-2}).
void legendre_pair(int m, double x, double& pm, double& pm1) {
    double a = 1.0, b = x;   // P_0, P_1
    if (m == 0) {
        pm = 1.0;
        pm1 = 0.0;
        return;
    }
    for (int k = 2; k <= m; ++k) {
        const double c = ((2.0 * k - 1.0) * x * b - (k - 1.0) * a) / double(k);
        a = b;
        b = c;
    }
    pm = b;
    pm1 = a;
}

// Nodes x_i = cos(theta_i), descending (colatitude ascending), and weights of
// a latitude grid's rule for the integral over [-1, 1]; theta_i as well, exact
// for the equiangular node sets.  The Gauss and Lobatto nodes are found by
// Newton's method from the usual cosine estimates, the first half only, and
// mirrored, so that the rule is exactly symmetric.
struct LatRule {
    std::vector<double> x, w, theta;
};

LatRule lat_rule(int grid, int n) {
    LatRule R;
    R.x.assign(n, 0.0);
    R.w.assign(n, 0.0);
    R.theta.assign(n, 0.0);
    if (grid == DISCO_GRID_EQUIANGULAR || grid == DISCO_GRID_EQUIANGULAR_TRAPEZOIDAL) {
        for (int i = 0; i < n; ++i) {
            R.theta[i] = kPi * double(i) / double(n - 1);
            R.x[i] = std::cos(R.theta[i]);
        }
        if (grid == DISCO_GRID_EQUIANGULAR) {
            R.w = clenshaw_curtis(n);
        } else {
            for (int i = 0; i + 1 < n; ++i) {   // trapezoid on [x_{i+1}, x_i]
                const double h = R.x[i] - R.x[i + 1];
                R.w[i] += 0.5 * h;
                R.w[i + 1] += 0.5 * h;
            }
        }
        return R;
    }
    if (grid == DISCO_GRID_LEGENDRE_GAUSS) {
        // roots of P_n; w = 2 / ((1 - x^2) P_n'(x)^2), P_n' = n (x P_n - P_{n-1}) / (x^2 - 1)
        for (int i = 0; i < (n + 1) / 2; ++i) {
            double x = std::cos(kPi * (i + 0.75) / (n + 0.5));
            double dp = 1.0;
            for (int it = 0; it < 100; ++it) {
                double p, p1;
                legendre_pair(n, x, p, p1);
                dp = double(n) * (x * p - p1) / (x * x - 1.0);
                const double dx = p / dp;
                x -= dx;
                if (std::fabs(dx) < 1e-16) break;
            }
            {
                double p, p1;
                legendre_pair(n, x, p, p1);
                dp = double(n) * (x * p - p1) / (x * x - 1.0);
            }
            if (2 * i + 1 == n) x = 0.0;   // the middle node of an odd rule
            const double w = 2.0 / ((1.0 - x * x) * dp * dp);
            R.x[i] = x;
            R.x[n - 1 - i] = -x;
            R.w[i] = R.w[n - 1 - i] = w;
        }
    } else {   // DISCO_GRID_LOBATTO: x = +-1 and the roots of P_{n-1}'
        const int m = n - 1;
        R.x[0] = 1.0;
        R.x[n - 1] = -1.0;
        R.w[0] = R.w[n - 1] = 2.0 / (double(n) * double(m));
        for (int i = 1; i < (n + 1) / 2; ++i) {
            double x = std::cos(kPi * double(i) / double(m));
            for (int it = 0; it < 100; ++it) {
                double p, p1;
                legendre_pair(m, x, p, p1);
                const double d1 = double(m) * (x * p - p1) / (x * x - 1.0);   // P_m'
                // Legendre's equation: (1 - x^2) P_m'' = 2 x P_m' - m (m + 1) P_m
                const double d2 = (2.0 * x * d1 - double(m) * (m + 1.0) * p) / (1.0 - x * x);
                const double dx = d1 / d2;
                x -= dx;
                if (std::fabs(dx) < 1e-16) break;
            }
            if (2 * i + 1 == n) x = 0.0;
            double p, p1;
            legendre_pair(m, x, p, p1);
            const double w = 2.0 / (double(n) * double(m) * p * p);
            R.x[i] = x;
            R.x[n - 1 - i] = -x;
            R.w[i] = R.w[n - 1 - i] = w;
        }
    }
    for (int i = 0; i < n; ++i) R.theta[i] = std::acos(R.x[i]);
    return R;
}

inline double hat(double u, double centre, double half_width) {
    const double v = 1.0 - std::fabs(u - centre) / half_width;
    return v > 0.0 ? v : 0.0;
}

struct Basis {
    int nr, nphi, K;
    double cutoff, dr;
    // Fills out[0..K) with the basis values at (r, alpha).
    void eval(double r, double alpha, double* out) const {
        double radial[kMaxK];
        for (int n = 0; n < nr; ++n) radial[n] = (nr == 1) ? 1.0 : hat(r, n * dr, dr);
        if (nphi == 0) {
            for (int n = 0; n < nr; ++n) out[n] = radial[n];
            return;
        }
        out[0] = radial[0];
        const double width = 2.0 * kPi / double(nphi);
        for (int m = 0; m < nphi; ++m) {
            double az = 1.0;
            if (nphi > 1) {
                double d = std::fmod(alpha - m * width, 2.0 * kPi);
                if (d < 0.0) d += 2.0 * kPi;
                if (d > kPi) d = 2.0 * kPi - d;   // circular distance
                az = hat(d, 0.0, width);
            }
            for (int n = 1; n < nr; ++n) out[1 + (n - 1) * nphi + m] = radial[n] * az;
        }
    }
};

bool is_nan(double v) { return v != v; }

}  // namespace

int build_host_psi(const disco_psi_desc& d, HostPsi& P) {
    if (d.nlat_in < 2 || d.nlat_out < 2)
        return set_error(DISCO_EINVAL, "nlat_in and nlat_out must be >= 2 (got %d, %d)",
                         d.nlat_in, d.nlat_out);
    if (d.nlon_in < 1 || d.nlon_out < 1)
        return set_error(DISCO_EINVAL, "nlon_in and nlon_out must be >= 1 (got %d, %d)",
                         d.nlon_in, d.nlon_out);
    if (d.nlon_out > d.nlon_in || d.nlon_in % d.nlon_out != 0)
        return set_error(DISCO_EINVAL,
                         "nlon_in (%d) must be a multiple of nlon_out (%d): the output "
                         "longitudes must be a subset of the input longitudes",
                         d.nlon_in, d.nlon_out);
    if ((int64_t)d.nlat_in * d.nlon_in > (int64_t)1 << 30 ||
        (int64_t)d.nlat_out * d.nlon_out > (int64_t)1 << 30)
        return set_error(DISCO_EUNSUPPORTED, "grid with more than 2^30 points");
    if (d.nlon_in > 65536)
        return set_error(DISCO_EUNSUPPORTED, "nlon_in > 65536");
    if (d.grid_in < DISCO_GRID_EQUIANGULAR || d.grid_in > DISCO_GRID_EQUIANGULAR_TRAPEZOIDAL ||
        d.grid_out < DISCO_GRID_EQUIANGULAR || d.grid_out > DISCO_GRID_EQUIANGULAR_TRAPEZOIDAL)
        return set_error(DISCO_EUNSUPPORTED, "unknown grid (got %d, %d)", d.grid_in, d.grid_out);
    if (d.basis_type != DISCO_BASIS_PIECEWISE_LINEAR)
        return set_error(DISCO_EUNSUPPORTED, "only the piecewise-linear basis is implemented");
    if (d.basis_norm != DISCO_NORM_NONE)
        return set_error(DISCO_EUNSUPPORTED, "only basis_norm = none is implemented");
    const int nr = d.kernel_shape[0], nphi = d.kernel_shape[1];
    if (nr < 1 || nphi < 0)
        return set_error(DISCO_EINVAL, "kernel_shape must have nr >= 1 and nphi >= 0 (got %d, %d)",
                         nr, nphi);
    const int64_t K64 = nphi == 0 ? nr : 1 + (int64_t)(nr - 1) * nphi;
    if (K64 > kMaxK || nr > kMaxK)
        return set_error(DISCO_EUNSUPPORTED, "K = %lld basis functions exceeds the limit of %d",
                         (long long)K64, kMaxK);
    double cutoff = d.theta_cutoff;
    if (is_nan(cutoff)) return set_error(DISCO_EINVAL, "theta_cutoff is NaN");
    if (cutoff <= 0.0) cutoff = double(nr + 1) * kPi / double(d.nlat_out - 1);
    if (!(cutoff < kPi))
        return set_error(DISCO_EINVAL, "theta_cutoff must be below pi (got %.17g)", cutoff);

    if (std::getenv("DISCO_TEST_FAIL_HOST_ALLOC"))
        return set_error(DISCO_ENOMEM, "host allocation failed (forced by DISCO_TEST_FAIL_HOST_ALLOC)");

    try {
        P.desc = d;
        P.cutoff = cutoff;
        P.nr = nr;
        P.nphi = nphi;
        P.K = int(K64);
        P.stride = d.nlon_in / d.nlon_out;
        const int K = P.K;
        Basis basis{nr, nphi, K, cutoff, nr > 1 ? cutoff / double(nr - 1) : cutoff};

        const LatRule rin = lat_rule(d.grid_in, d.nlat_in);
        const LatRule rout = lat_rule(d.grid_out, d.nlat_out);
        const std::vector<double>& wcc = rin.w;
        const std::vector<double>& th_in = rin.theta;
        std::vector<double> cos_in(d.nlat_in), sin_in(d.nlat_in);
        for (int i = 0; i < d.nlat_in; ++i) {
            cos_in[i] = std::cos(th_in[i]);
            sin_in[i] = std::sin(th_in[i]);
        }
        std::vector<double> cos_lam(d.nlon_in), sin_lam(d.nlon_in);
        for (int p = 0; p < d.nlon_in; ++p) {
            const double lam = 2.0 * kPi * double(p) / double(d.nlon_in);
            cos_lam[p] = std::cos(lam);
            sin_lam[p] = std::sin(lam);
        }
        const double lon_weight = 2.0 * kPi / double(d.nlon_in);
        const double limit = cutoff * (1.0 - kTieRel);

        P.row_ptr.assign(d.nlat_out + 1, 0);
        P.win_ptr.assign(d.nlat_out + 1, 0);
        P.in_lat.clear();
        P.lon_off.clear();
        P.vals.clear();
        P.windows.clear();
        P.win_vals.clear();
        P.nnz_nonzero = 0;

        std::vector<double> r(d.nlon_in), alpha(d.nlon_in);
        std::vector<char> inside(d.nlon_in);
        std::vector<double> bv(K);
        for (int j = 0; j < d.nlat_out; ++j) {
            const double tho = rout.theta[j];
            // unit vector of the output point and its local south/east axes
            const double ax = std::sin(tho), az = std::cos(tho);
            const double sx = std::cos(tho), sz = -std::sin(tho);   // south; east = (0,1,0)
            for (int i = 0; i < d.nlat_in; ++i) {
                if (std::fabs(th_in[i] - tho) > cutoff * (1.0 + 1e-9)) continue;
                const double om = wcc[i] * lon_weight;
                int count = 0;
                for (int p = 0; p < d.nlon_in; ++p) {
                    const double bx = sin_in[i] * cos_lam[p];
                    const double by = sin_in[i] * sin_lam[p];
                    const double bz = cos_in[i];
                    const double u = bx * sx + bz * sz;       // component along local south
                    const double v = by;                      // component along local east
                    const double c = bx * ax + bz * az;       // along the output point
                    r[p] = std::atan2(std::sqrt(u * u + v * v), c);
                    double a = std::atan2(v, u);
                    if (a < 0.0) a += 2.0 * kPi;
                    alpha[p] = a;
                    inside[p] = r[p] < limit;
                    count += inside[p];
                }
                if (count == 0) continue;
                // canonical entries, ascending longitude
                for (int p = 0; p < d.nlon_in; ++p) {
                    if (!inside[p]) continue;
                    basis.eval(r[p], alpha[p], bv.data());
                    P.in_lat.push_back(i);
                    P.lon_off.push_back(p);
                    for (int k = 0; k < K; ++k) {
                        P.vals.push_back(bv[k] * om);
                        if (bv[k] > 1e-12) ++P.nnz_nonzero;
                    }
                }
                // window: one circular interval of longitudes
                int p_lo = 0;
                if (count < d.nlon_in) {
                    p_lo = -1;
                    for (int p = 0; p < d.nlon_in; ++p) {
                        const int prev = (p + d.nlon_in - 1) % d.nlon_in;
                        if (inside[p] && !inside[prev]) {
                            if (p_lo >= 0)
                                return set_error(DISCO_EUNSUPPORTED,
                                                 "support of output row %d in input row %d is not "
                                                 "one longitude interval", j, i);
                            p_lo = p;
                        }
                    }
                }
                Window wnd;
                wnd.lat = i;
                wnd.p_lo = p_lo;
                wnd.width = count;
                wnd.val_off = (int64_t)(P.win_vals.size() / K);
                for (int t = 0; t < count; ++t) {
                    const int p = (p_lo + t) % d.nlon_in;
                    basis.eval(r[p], alpha[p], bv.data());
                    for (int k = 0; k < K; ++k) P.win_vals.push_back(bv[k] * om);
                }
                P.windows.push_back(wnd);
            }
            P.row_ptr[j + 1] = (int64_t)P.in_lat.size();
            P.win_ptr[j + 1] = (int64_t)P.windows.size();
        }
        if (P.in_lat.size() > (size_t)0x7fffffff)
            return set_error(DISCO_EUNSUPPORTED, "more than 2^31 support points");
    } catch (const std::bad_alloc&) {
        return set_error(DISCO_ENOMEM, "host allocation failed while building Psi");
    }
    return DISCO_OK;
}

}  // namespace disco
