// Complex helpers and the register-resident DFTs of the longitude-spectral
// kernels.  Everything here is __host__ __device__, so the same templates can
// be compiled for the CPU and checked there against a float64 DFT.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

namespace disco {
namespace specdft {

__host__ __device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__host__ __device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__host__ __device__ __forceinline__ float2 cscale(float2 a, float s) { return make_float2(a.x * s, a.y * s); }
__host__ __device__ __forceinline__ float2 cmul(float2 a, float2 b) {
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
__host__ __device__ __forceinline__ float2 cconj(float2 a) { return make_float2(a.x, -a.y); }
// i * s * a for s = +-1
__host__ __device__ __forceinline__ float2 cimul(float2 a, float s) { return make_float2(-s * a.y, s * a.x); }

// In-place DFT of length R: a[u] <- sum_t a[t] exp(s * 2 pi i u t / R).
template <int R>
__host__ __device__ __forceinline__ void butterfly(float2 (&a)[R], float s);

template <>
__host__ __device__ __forceinline__ void butterfly<2>(float2 (&a)[2], float) {
    const float2 t = a[0];
    a[0] = cadd(t, a[1]);
    a[1] = csub(t, a[1]);
}

template <>
__host__ __device__ __forceinline__ void butterfly<4>(float2 (&a)[4], float s) {
    const float2 p0 = cadd(a[0], a[2]), p1 = cadd(a[1], a[3]);
    const float2 t1 = csub(a[0], a[2]), t2 = cimul(csub(a[1], a[3]), s);
    a[0] = cadd(p0, p1);
    a[1] = cadd(t1, t2);
    a[2] = csub(p0, p1);
    a[3] = csub(t1, t2);
}

template <>
__host__ __device__ __forceinline__ void butterfly<3>(float2 (&a)[3], float s) {
    const float2 t = cadd(a[1], a[2]), d = csub(a[1], a[2]);
    const float2 m = csub(a[0], cscale(t, 0.5f));
    const float2 e = cimul(cscale(d, 0.86602540378443865f), s);
    a[0] = cadd(a[0], t);
    a[1] = cadd(m, e);
    a[2] = csub(m, e);
}

template <>
__host__ __device__ __forceinline__ void butterfly<5>(float2 (&a)[5], float s) {
    const float c1 = 0.30901699437494742f, c2 = -0.80901699437494742f;
    const float s1 = 0.95105651629515357f, s2 = 0.58778525229247313f;
    const float2 t1 = cadd(a[1], a[4]), t2 = cadd(a[2], a[3]);
    const float2 d1 = csub(a[1], a[4]), d2 = csub(a[2], a[3]);
    const float2 r1 = cadd(a[0], cadd(cscale(t1, c1), cscale(t2, c2)));
    const float2 r2 = cadd(a[0], cadd(cscale(t1, c2), cscale(t2, c1)));
    const float2 i1 = cimul(cadd(cscale(d1, s1), cscale(d2, s2)), s);
    const float2 i2 = cimul(csub(cscale(d1, s2), cscale(d2, s1)), s);
    a[0] = cadd(a[0], cadd(t1, t2));
    a[1] = cadd(r1, i1);
    a[4] = csub(r1, i1);
    a[2] = cadd(r2, i2);
    a[3] = csub(r2, i2);
}


// ---------------------------------------------------------------------------
// Register-resident transforms for N/2 = H1 * H2 (a four-step split of the
// complex transform, each step's short DFTs unrolled in registers).

// Compile-time cosine and sine: Taylor series after reduction to [-pi, pi]
// (through degree 31, far below float rounding there).
constexpr double kPiD = 3.14159265358979323846;
constexpr double ct_reduce(double x) {
    while (x > kPiD) x -= 2.0 * kPiD;
    while (x < -kPiD) x += 2.0 * kPiD;
    return x;
}
constexpr double ct_sin(double x) {
    x = ct_reduce(x);
    double term = x, sum = x;
    for (int n = 1; n < 16; ++n) {
        term *= -x * x / ((2.0 * n) * (2.0 * n + 1.0));
        sum += term;
    }
    return sum;
}
constexpr double ct_cos(double x) {
    x = ct_reduce(x);
    double term = 1.0, sum = 1.0;
    for (int n = 1; n < 16; ++n) {
        term *= -x * x / ((2.0 * n - 1.0) * (2.0 * n));
        sum += term;
    }
    return sum;
}

template <int I, int N, typename F>
__host__ __device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// v * exp(S * 2 pi i * E / N) for a compile-time exponent E
template <int N, int S, int E>
__host__ __device__ __forceinline__ float2 rot_ct(float2 v) {
    constexpr int e = ((E % N) + N) % N;
    if constexpr (e == 0) {
        return v;
    } else if constexpr (2 * e == N) {
        return make_float2(-v.x, -v.y);
    } else if constexpr (4 * e == N) {
        return cimul(v, (float)S);
    } else if constexpr (4 * e == 3 * N) {
        return cimul(v, (float)-S);
    } else {
        constexpr float c = (float)ct_cos(2.0 * kPiD * e / N);
        constexpr float sn = (float)(S * ct_sin(2.0 * kPiD * e / N));
        return cmul(v, make_float2(c, sn));
    }
}

// Prime-factor split of N: the largest power of 2, 3 or 5 dividing N that is
// not N itself and leaves a cofactor coprime to it (1 if there is none).
constexpr int pfa_factor(int n) {
    for (int p : {2, 3, 5}) {
        int q = 1;
        while (n % (q * p) == 0) q *= p;
        if (q > 1 && q < n) return q;
    }
    return 1;
}
// x with (x * a) % m == 1 (a and m coprime)
constexpr int inverse_mod(int a, int m) {
    for (int x = 1; x < m; ++x)
        if ((x * a) % m == 1) return x;
    return 1;
}

// In-place DFT of length N in registers, a[u] <- sum_t a[t] exp(S 2 pi i u t / N),
// every index and root compile-time.  Coprime factors N = N1 N2 take the
// prime-factor algorithm (Good 1958, Thomas 1963): input index
// (N2 n1 + N1 n2) mod N, output index (N2 T1 k1 + N1 T2 k2) mod N with
// T1 = N2^-1 mod N1, T2 = N1^-1 mod N2, and no twiddle factors between the
// two sets of short DFTs.  Prime powers use mixed-radix decimation in time
// (radix 4, 2, 3, 5 first).
template <int N, int S>
__host__ __device__ __forceinline__ void reg_dft(float2 (&a)[N]) {
    if constexpr (N == 1) {
    } else if constexpr (N <= 5) {
        butterfly<N>(a, (float)S);
    } else if constexpr (pfa_factor(N) > 1) {
        constexpr int N1 = pfa_factor(N), N2 = N / N1;
        constexpr int T1 = inverse_mod(N2 % N1, N1), T2 = inverse_mod(N1 % N2, N2);
        float2 y[N2][N1];
        static_for<0, N2>([&](auto n2) {
            static_for<0, N1>([&](auto n1) { y[n2][n1] = a[(N2 * n1 + N1 * n2) % N]; });
            reg_dft<N1, S>(y[n2]);
        });
        static_for<0, N1>([&](auto k1) {
            float2 t[N2];
            static_for<0, N2>([&](auto n2) { t[n2] = y[n2][k1]; });
            reg_dft<N2, S>(t);
            static_for<0, N2>([&](auto k2) { a[(N2 * T1 * k1 + N1 * T2 * k2) % N] = t[k2]; });
        });
    } else {
        constexpr int R = N % 4 == 0 ? 4 : N % 2 == 0 ? 2 : N % 3 == 0 ? 3 : 5;
        constexpr int M = N / R;
        static_assert(R * M == N && N % R == 0, "N must be a product of 2, 3 and 5");
        float2 y[R][M];
        static_for<0, R>([&](auto r) {
            static_for<0, M>([&](auto m) { y[r][m] = a[R * m + r]; });
            reg_dft<M, S>(y[r]);
        });
        // X[k1 + M k2] = sum_r exp(S 2 pi i r k1 / N) exp(S 2 pi i r k2 / R) Y_r[k1]
        static_for<0, M>([&](auto k1) {
            float2 t[R];
            static_for<0, R>([&](auto r) {
                t[r] = rot_ct<N, S, decltype(r)::value * decltype(k1)::value>(y[r][k1]);
            });
            butterfly<R>(t, (float)S);
            static_for<0, R>([&](auto k2) { a[k1 + M * k2] = t[k2]; });
        });
    }
}


}  // namespace specdft
}  // namespace disco
