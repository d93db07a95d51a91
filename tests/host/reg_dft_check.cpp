// CPU check of the register-resident DFTs used by the longitude-spectral
// kernels: the same templates (spectral_dft.h), compiled for the host, against
// the discrete Fourier transform evaluated from its definition in float64.
// Prints one line per (length, sign): "N S max_abs_err max_rel_err", where the
// relative error is the largest absolute error over the largest |X| of the
// exact transform.  Inputs are seeded uniform values in [-1, 1).
#include <cmath>
#include <cstdint>
#include <cstdio>

#include "spectral_dft.h"

using disco::specdft::reg_dft;

static uint64_t g_state = 0x9e3779b97f4a7c15ull;
static double next_uniform() {   // splitmix64 -> [-1, 1)
    uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (double)(z >> 11) * (1.0 / 9007199254740992.0) * 2.0 - 1.0;
}

template <int N, int S>
static int check(int trials) {
    double max_abs = 0.0, max_ref = 0.0;
    for (int t = 0; t < trials; ++t) {
        float2 a[N];
        double re[N], im[N];
        for (int n = 0; n < N; ++n) {
            a[n] = make_float2((float)next_uniform(), (float)next_uniform());
            re[n] = a[n].x;
            im[n] = a[n].y;
        }
        reg_dft<N, S>(a);
        for (int u = 0; u < N; ++u) {
            double xr = 0.0, xi = 0.0;
            for (int n = 0; n < N; ++n) {
                // exp(S 2 pi i u n / N), the exponent reduced exactly first
                const double ang = S * 2.0 * M_PI * (double)((int64_t)u * n % N) / N;
                xr += re[n] * std::cos(ang) - im[n] * std::sin(ang);
                xi += re[n] * std::sin(ang) + im[n] * std::cos(ang);
            }
            const double e = std::hypot(a[u].x - xr, a[u].y - xi);
            if (e > max_abs) max_abs = e;
            const double m = std::hypot(xr, xi);
            if (m > max_ref) max_ref = m;
        }
    }
    std::printf("%d %d %.3e %.3e\n", N, S, max_abs, max_abs / max_ref);
    return 0;
}

template <int N>
static void both(int trials) {
    check<N, -1>(trials);
    check<N, 1>(trials);
}

int main() {
    // the short lengths the kernels instantiate (four-step factors of the
    // 720-, 360- and 180-point half-length transforms) and the radices and
    // prime-factor splits they are built from
    both<2>(64);
    both<3>(64);
    both<4>(64);
    both<5>(64);
    both<8>(64);
    both<9>(64);
    both<15>(64);
    both<16>(64);
    both<25>(64);
    both<45>(64);
    both<32>(16);
    both<60>(16);
    both<90>(8);
    return 0;
}
