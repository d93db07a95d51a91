// Longitude-spectral form of Psi, for layers with equal input and output
// longitude counts (stride 1).
//
// With stride 1 the forward equation's inner sum over one output row j and
// one input row i is a circular correlation along longitude (the p-shift of
// the DiscreteContinuousConvS2 page): with the window's values v[k, t] at
// longitudes p = p_lo + t,
//   X_K[k, q] = sum_t v[k, t] * x[(q + p_lo + t) mod N].
// Its discrete Fourier transform over q is conj(Psi_hat[k, m]) * x_hat[m]
// with Psi_hat[k, m] = sum_t v[k, t] * exp(-2 pi i m (p_lo + t) / N).  x is
// real, so frequencies m = 0 .. N/2 carry everything.
//
// This file tabulates, in float64:
//   * Psi_hat per window for m < N/2 + 1, zero up to the padded count MP
//     (a multiple of 32), stored as bf16 (re, im) pairs in one 32-bit word
//     (real part in the low half): the matrix-core operand type it feeds;
//     and, for stride 1 when it takes at most 256 MiB, as float32 pairs for
//     float32 layers;
//   * the radix plan (4, 2, 3, 5) of the N/2-point complex transform the
//     real transforms are built on.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <atomic>
#include <functional>
#include <thread>
#include <vector>

#include "disco_internal.h"

namespace disco {

bool parallel_ranges(size_t n, const std::function<void(size_t, size_t)>& fn) {
    const unsigned hw = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    const size_t per = (n + hw - 1) / hw;
    std::atomic<bool> ok{true};
    auto run = [&](size_t a, size_t b) {
        try {
            fn(a, b);
        } catch (...) {
            ok = false;
        }
    };
    std::vector<std::thread> pool;
    std::vector<std::pair<size_t, size_t>> left;   // shares no thread could take
    for (unsigned t = 0; t < hw; ++t) {
        const size_t a = t * per, b = std::min(n, a + per);
        if (a >= b) continue;
        try {
            pool.emplace_back(run, a, b);
        } catch (...) {   // std::system_error (thread limit) or bad_alloc
            left.emplace_back(a, b);
        }
    }
    for (const auto& r : left) run(r.first, r.second);
    for (auto& th : pool) th.join();
    return ok;
}


namespace {

// double -> bf16, round to nearest even.  The intermediate float is rounded to
// odd (inexact results get their lowest bit set), so the second rounding sees
// the sticky information of the first and the result is the correctly rounded
// bf16 of the double.
uint32_t bf16_of(double v) {
    float f = (float)v;
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((double)f != v && std::isfinite(f)) {
        // back to round-toward-zero, then set the sticky bit
        if (std::fabs((double)f) > std::fabs(v)) u -= 1;
        u |= 1u;
    }
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

}  // namespace

int spectral_plan(int n, int32_t* radix, int32_t* nrad) {
    int cnt = 0;
    for (int r : {4, 2, 3, 5}) {
        while (n % r == 0 && cnt < kSpecMaxRadix) {
            radix[cnt++] = r;
            n /= r;
        }
    }
    *nrad = cnt;
    return n == 1;
}

int build_spectral_tables(const HostPsi& h, std::vector<uint32_t>& psih, std::vector<float>& psih32,
                          int32_t* radix, int32_t* nrad, int32_t* mp) {
    *mp = 0;
    psih32.clear();
    *nrad = 0;
    const int N = h.desc.nlon_in;
    // stride 1; or stride 2 where both transforms have register forms (input
    // halves of 720 and 360 points): the stride-2 output is the stride-1
    // correlation at every second longitude, folded in the frequency domain
    const bool s1 = h.stride == 1 && h.desc.nlon_out == N;
    const bool s2 = h.stride == 2 && (N == 1440 || N == 720);
    if ((!s1 && !s2) || N % 2 != 0 || N < 4 || N > kSpecMaxN || h.K > 8 ||
        !spectral_plan(N / 2, radix, nrad))
        return DISCO_OK;   // not eligible: no tables
    const int M = N / 2 + 1;
    const int MP = (M + 31) / 32 * 32;
    const int K = h.K;
    const size_t nwin = h.windows.size();
    std::vector<double> c(N), s(N);
    for (int n = 0; n < N; ++n) {
        const double a = 2.0 * M_PI * (double)n / (double)N;
        c[n] = std::cos(a);
        s[n] = std::sin(a);
    }
    // the float32 table (float32 layers, stride 1) when it takes at most 256 MiB
    const bool f32 = s1 && nwin * (size_t)K * MP * 8 <= ((size_t)256 << 20);
    try {
        // plus a zero block of 32 words at the end (a DMA source for the
        // slices of windows a row does not have)
        psih.assign(nwin * (size_t)K * MP + 32, 0u);
        if (f32) psih32.assign(nwin * (size_t)K * MP * 2, 0.0f);
    } catch (const std::bad_alloc&) {
        return set_error(DISCO_ENOMEM, "host allocation for the spectral tables failed");
    }
    auto work = [&](size_t w0, size_t w1) {
        std::vector<double> re(K), im(K);
        for (size_t w = w0; w < w1; ++w) {
            const Window& wd = h.windows[w];
            const double* v = h.win_vals.data() + (size_t)wd.val_off * K;
            for (int m = 0; m < M; ++m) {
                std::fill(re.begin(), re.end(), 0.0);
                std::fill(im.begin(), im.end(), 0.0);
                for (int t = 0; t < wd.width; ++t) {
                    int p = (wd.p_lo + t) % N;
                    if (p < 0) p += N;
                    const int e = (int)(((int64_t)m * p) % N);
                    for (int k = 0; k < K; ++k) {
                        re[k] += v[(size_t)t * K + k] * c[e];
                        im[k] -= v[(size_t)t * K + k] * s[e];
                    }
                }
                for (int k = 0; k < K; ++k) {
                    const size_t e = (w * K + k) * (size_t)MP + m;
                    psih[e] = bf16_of(re[k]) | (bf16_of(im[k]) << 16);
                    if (f32) {
                        psih32[2 * e] = (float)re[k];
                        psih32[2 * e + 1] = (float)im[k];
                    }
                }
            }
        }
    };
    if (!parallel_ranges(nwin, work))
        return set_error(DISCO_ENOMEM, "host allocation for the spectral tables failed");
    *mp = MP;
    return DISCO_OK;
}

}  // namespace disco
