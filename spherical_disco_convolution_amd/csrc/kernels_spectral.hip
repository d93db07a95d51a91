// Spectral evaluation of the fused DISCO forward pass for stride-1 layers.
//
// Along longitude the forward equation's inner sum is, per (output row,
// input row) window, a circular correlation (the p-shift of the
// DiscreteContinuousConvS2 page).  With the real DFT over longitude,
//   X_hat[b,ci,k,j,m] = sum_windows x_hat[b,ci,i,m] * conj(Psi_hat[k,j,i,m])
//   y_hat[b,co,j,m]   = sum_{ci,k} w[co,ci,k] * X_hat[b,ci,k,j,m]
//   y[b,co,j,:]       = inverse real DFT of y_hat[b,co,j,:] (+ bias)
// (the channel and basis sums of the forward equation commute with the DFT).
// Psi_hat comes from spectral_host.cpp.  Three kernels:
//   spec_rfft   x rows -> x_hat, stored as bf16 (re, im) pairs;
//   spec_mfma   per (batch, output row, 32 frequencies): the window sum on
//               the matrix cores into a bf16 [frequency, re/im][(ci, k)] LDS
//               tile per 32-channel chunk, then the channel/basis GEMM on
//               v_mfma_f32_32x32x16_bf16 into y_hat (bf16 pairs);
//   spec_irfft  y_hat rows -> y rows (+ bias).
// The real transforms run an N/2-point complex transform in LDS: iterative
// Stockham passes of radix 4, 2, 3 and 5 (Govindaraju et al., "High
// performance discrete Fourier transforms on graphics processors", SC 2008),
// with the usual packing of even and odd samples into one complex sequence.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "disco_internal.h"
#include "kernels_common.h"

namespace disco {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct SpecPlan {
    int32_t n;
    int32_t r[kSpecMaxRadix];
};

__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cscale(float2 a, float s) { return make_float2(a.x * s, a.y * s); }
__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
__device__ __forceinline__ float2 cconj(float2 a) { return make_float2(a.x, -a.y); }
// i * s * a for s = +-1
__device__ __forceinline__ float2 cimul(float2 a, float s) { return make_float2(-s * a.y, s * a.x); }

// In-place DFT of length R: a[u] <- sum_t a[t] exp(s * 2 pi i u t / R).
template <int R>
__device__ __forceinline__ void butterfly(float2 (&a)[R], float s);

template <>
__device__ __forceinline__ void butterfly<2>(float2 (&a)[2], float) {
    const float2 t = a[0];
    a[0] = cadd(t, a[1]);
    a[1] = csub(t, a[1]);
}

template <>
__device__ __forceinline__ void butterfly<4>(float2 (&a)[4], float s) {
    const float2 p0 = cadd(a[0], a[2]), p1 = cadd(a[1], a[3]);
    const float2 t1 = csub(a[0], a[2]), t2 = cimul(csub(a[1], a[3]), s);
    a[0] = cadd(p0, p1);
    a[1] = cadd(t1, t2);
    a[2] = csub(p0, p1);
    a[3] = csub(t1, t2);
}

template <>
__device__ __forceinline__ void butterfly<3>(float2 (&a)[3], float s) {
    const float2 t = cadd(a[1], a[2]), d = csub(a[1], a[2]);
    const float2 m = csub(a[0], cscale(t, 0.5f));
    const float2 e = cimul(cscale(d, 0.86602540378443865f), s);
    a[0] = cadd(a[0], t);
    a[1] = cadd(m, e);
    a[2] = csub(m, e);
}

template <>
__device__ __forceinline__ void butterfly<5>(float2 (&a)[5], float s) {
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

// exp(s * 2 pi i * e / H), with the hardware sine and cosine (|angle| <= 2 pi)
__device__ __forceinline__ float2 root(int e, float inv_h, float s) {
    float sn, cs;
    __sincosf(6.28318530717958648f * (float)e * inv_h, &sn, &cs);
    return make_float2(cs, s * sn);
}

// The wave's LDS accesses are complete (and the compiler keeps later LDS
// accesses after this point): enough between the steps of a transform that
// one wave owns.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// One in-place Stockham pass of radix R over an H-point sequence whose
// sub-transforms of length Ns are done, by the 64 lanes of one wave (s = -1
// forward, +1 inverse).  The lane's butterflies j = lane + 64 it (at most MAXIT)
// first read all their inputs into registers, then wait for those reads, then
// write: so one buffer per row suffices.  Quotients by Ns use a float
// reciprocal: (j + 1/2) / Ns is below H / 2 and at least 1 / (2 Ns) >= 1 / H
// from an integer, and the float product is within 2 ulp of it (H <= 900), so
// truncation gives the exact quotient.
template <int R, int MAXIT>
__device__ __forceinline__ void stockham_pass(float2* buf, int H, int Ns, const float2* twl,
                                              float s, int lane) {
    const int HR = H / R;
    const int ts = H / (Ns * R);
    const float inv_ns = 1.0f / (float)Ns;
    float2 a[MAXIT][R];
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
        const int j = lane + 64 * it;
        if (j < HR) {
#pragma unroll
            for (int t = 0; t < R; ++t) a[it][t] = buf[j + t * HR];
        }
    }
    wave_lds_sync();
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
        const int j = lane + 64 * it;
        if (j < HR) {
            const int q = (int)(((float)j + 0.5f) * inv_ns);
            const int jj = j - q * Ns;
            if (jj != 0) {
                // twl[e] = exp(-2 pi i e / H); e = jj * t * ts < H
#pragma unroll
                for (int t = 1; t < R; ++t) {
                    float2 w = twl[jj * t * ts];
                    if (s > 0.0f) w.y = -w.y;
                    a[it][t] = cmul(a[it][t], w);
                }
            }
            butterfly<R>(a[it], s);
            const int base = q * Ns * R + jj;
#pragma unroll
            for (int u = 0; u < R; ++u) buf[base + u * Ns] = a[it][u];
        }
    }
    wave_lds_sync();
}

// H-point complex DFT, in place in buf (one wave's LDS row), with the
// workgroup's twiddle table twl[e] = exp(-2 pi i e / H).  The transform
// belongs to one wave, so passes are separated by wave-level waits.
// H <= kSpecMaxN / 2 = 900 bounds the butterflies per lane (MAXIT).
__device__ void fft_wave(float2* buf, int H, const SpecPlan& pl, const float2* twl, float s,
                         int lane) {
    int Ns = 1;
    for (int p = 0; p < pl.n; ++p) {
        switch (pl.r[p]) {
            case 4: stockham_pass<4, 4>(buf, H, Ns, twl, s, lane); break;
            case 2: stockham_pass<2, 8>(buf, H, Ns, twl, s, lane); break;
            case 3: stockham_pass<3, 5>(buf, H, Ns, twl, s, lane); break;
            default: stockham_pass<5, 3>(buf, H, Ns, twl, s, lane); break;
        }
        Ns *= pl.r[p];
    }
}

typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// two floats -> bf16 pair (round to nearest even, one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v){lo, hi}, bf16x2v));
}

constexpr int kFftThreads = 256;
constexpr int kFftRows = kFftThreads / 64;   // one wave per row

// Twiddle table of the workgroup: twl[e] = exp(-2 pi i e / H), e < H.
__device__ __forceinline__ void fill_twiddles(float2* twl, int H) {
    const float inv_h = 1.0f / (float)H;
    for (int e = threadIdx.x; e < H; e += blockDim.x) twl[e] = root(e, inv_h, -1.0f);
}

// x rows (N real, bf16) -> x_hat rows (MP bf16 pairs; frequencies past N/2
// are zero).  One wave per row, four rows per workgroup; LDS: one H-point
// buffer per row and the H-point twiddle table.  Waves past the last row
// leave after the table is built.
__global__ __launch_bounds__(kFftThreads) void spec_rfft(const bf16_t* __restrict__ x,
                                                         uint32_t* __restrict__ xh, int N, int MP,
                                                         int64_t nrows, SpecPlan pl) {
    extern __shared__ float2 sm[];
    const int H = N / 2;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kFftRows + wave;
    const bool live = row < nrows;
    float2* b0 = sm + (size_t)wave * H;
    float2* twl = sm + (size_t)kFftRows * H;
    fill_twiddles(twl, H);
    const uint32_t* xr = reinterpret_cast<const uint32_t*>(x + (live ? row : 0) * (size_t)N);
    for (int n = lane; n < H; n += 64) {
        const uint32_t v = xr[n];   // samples 2n (low half) and 2n + 1
        b0[n] = make_float2(__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u));
    }
    __syncthreads();   // the twiddle table
    if (!live) return;
    fft_wave(b0, H, pl, twl, -1.0f, lane);
    const float2* z = b0;
    // X[m] = (a + b)/2 - i W^m (a - b)/2, a = Z[m mod H], b = conj(Z[(H - m) mod H]),
    // W = exp(-2 pi i / N)
    uint32_t* out = xh + row * (size_t)MP;
    const float inv_n = 0.5f / (float)H;
    for (int m = lane; m < MP; m += 64) {
        float2 X = make_float2(0.0f, 0.0f);
        if (m <= H) {
            const float2 a = z[m == H ? 0 : m];
            const float2 b = cconj(z[m == 0 ? 0 : H - m]);
            const float2 e = cmul(root(m, inv_n, -1.0f), csub(a, b));
            X = cadd(cscale(cadd(a, b), 0.5f), cscale(make_float2(e.y, -e.x), 0.5f));
        }
        out[m] = pack_bf16x2(X.x, X.y);
    }
}

// y_hat rows (MP bf16 pairs, frequencies 0..N/2 used) -> y rows (N) + bias,
// one wave per row (LDS as for spec_rfft).  The imaginary parts of the zero and N/2 frequencies are
// dropped (a real row's spectrum has none).
template <typename TY>
__global__ __launch_bounds__(kFftThreads) void spec_irfft(const uint32_t* __restrict__ yh,
                                                          TY* __restrict__ y,
                                                          const float* __restrict__ bias, int N,
                                                          int MP, int Co, int nlat_out,
                                                          int64_t nrows, SpecPlan pl) {
    extern __shared__ float2 sm[];
    const int H = N / 2;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kFftRows + wave;
    const bool live = row < nrows;
    float2* b0 = sm + (size_t)wave * H;
    float2* twl = sm + (size_t)kFftRows * H;
    fill_twiddles(twl, H);
    const uint32_t* src = yh + (live ? row : 0) * (size_t)MP;
    auto spec = [&](int m) {
        const uint32_t v = src[m];
        return make_float2(__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u));
    };
    // Z[m] = (a + b)/2 + i conj(W^m) (a - b)/2, a = X[m], b = conj(X[H - m]), m < H
    const float inv_n = 0.5f / (float)H;
    for (int m = lane; m < H; m += 64) {
        float2 a = spec(m);
        float2 b = cconj(spec(H - m));
        if (m == 0) {
            a.y = 0.0f;
            b.y = 0.0f;
        }
        const float2 e = cmul(root(m, inv_n, 1.0f), csub(a, b));
        b0[m] = cadd(cscale(cadd(a, b), 0.5f), cscale(make_float2(-e.y, e.x), 0.5f));
    }
    __syncthreads();   // the twiddle table, b0
    if (!live) return;
    fft_wave(b0, H, pl, twl, 1.0f, lane);
    const float2* z = b0;
    const float bv = bias ? bias[(row / nlat_out) % Co] : 0.0f;
    const float sc = 1.0f / (float)H;
    TY* out = y + row * (size_t)N;
    for (int n = lane; n < H; n += 64) {
        const float2 v = z[n];
        if constexpr (sizeof(TY) == 4) {
            *reinterpret_cast<float2*>(out + 2 * n) = make_float2(v.x * sc + bv, v.y * sc + bv);
        } else {
            *reinterpret_cast<uint32_t*>(out + 2 * n) = pack_bf16x2(v.x * sc + bv, v.y * sc + bv);
        }
    }
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
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// v * exp(S * 2 pi i * E / N) for a compile-time exponent E
template <int N, int S, int E>
__device__ __forceinline__ float2 rot_ct(float2 v) {
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
__device__ __forceinline__ void reg_dft(float2 (&a)[N]) {
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

__device__ __forceinline__ float2 unpack_bf16x2(uint32_t v) {
    return make_float2(__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u));
}

constexpr int kRegThreads = 64;   // one wave per workgroup

constexpr int spec_mp_of(int H) { return (H + 32) / 32 * 32; }   // (H + 1) rounded up to 32

// x rows (N = 2 H real bf16 samples, H = H1 H2) -> x_hat rows (MP bf16 pairs),
// RW rows per wave and step.  The H-point transform of z[n] = x[2n] + i x[2n+1]
// is split with n = H2 a + b and k = c + H1 d:
//   step A, tasks (row, b): A[b, c] = w_H^{b c} sum_a z[H2 a + b] w_H1^{a c};
//   step B, tasks (row, c): Z[c + H1 d] = sum_b A[b, c] w_H2^{b d};
// w_L = exp(-2 pi i / L).  Step A reads its samples from memory (lanes b
// consecutive), A passes through LDS with a row stride P2 (odd, so step B's
// strided reads spread over the banks), Z returns to LDS in natural order for
// the even/odd split, which writes four frequencies per 16-byte store.
// Workgroup g transforms rows g RW .. g RW + RW - 1.  (A persistent form that
// loads the next group during the current one needs more than 256 registers
// and is slower.)
template <int H1, int H2, int RW>
__global__ __launch_bounds__(kRegThreads) void spec_rfft_reg(const uint32_t* __restrict__ x,
                                                             uint32_t* __restrict__ xh,
                                                             int64_t nrows) {
    constexpr int H = H1 * H2, MP = spec_mp_of(H);
    constexpr int P2 = H2 | 1, LP = H1 * P2;
    constexpr int TA = RW * H2, ITA = (TA + 63) / 64;
    constexpr int TB = RW * H1, ITB = (TB + 63) / 64;
    static_assert(LP >= H, "the split needs H entries per row");
    static_assert(MP - H - 1 <= 64, "one lane per padding word");
    __shared__ float2 buf[RW * LP];
    const int lane = threadIdx.x;
    const int64_t g = blockIdx.x;   // the grid is the row-group count

    uint32_t raw[ITA][H1];
#pragma unroll
    for (int i = 0; i < ITA; ++i) {
        const int t = min(lane + 64 * i, TA - 1);
        const int r = t / H2, b = t - r * H2;
        const int64_t row = min(g * RW + r, nrows - 1);
        const uint32_t* src = x + row * H + b;
#pragma unroll
        for (int a = 0; a < H1; ++a) raw[i][a] = src[H2 * a];
    }
    {
        // ---- step A ----
#pragma unroll
        for (int i = 0; i < ITA; ++i) {
            const int t = lane + 64 * i;
            const int tc = min(t, TA - 1);
            const int r = tc / H2, b = tc - r * H2;
            float2 v[H1];
#pragma unroll
            for (int a = 0; a < H1; ++a) v[a] = unpack_bf16x2(raw[i][a]);
            reg_dft<H1, -1>(v);
            const float2 w = root(b, 1.0f / (float)H, -1.0f);
            float2 p = w;
#pragma unroll
            for (int c = 1; c < H1; ++c) {
                v[c] = cmul(v[c], p);
                p = cmul(p, w);
            }
            if (t < TA) {
#pragma unroll
                for (int c = 0; c < H1; ++c) buf[r * LP + c * P2 + b] = v[c];
            }
        }
        wave_lds_sync();
        // ---- step B ----
        float2 v[ITB][H2];
#pragma unroll
        for (int i = 0; i < ITB; ++i) {
            const int t = min(lane + 64 * i, TB - 1);
            const int r = t / H1, c = t - r * H1;
#pragma unroll
            for (int b = 0; b < H2; ++b) v[i][b] = buf[r * LP + c * P2 + b];
        }
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < ITB; ++i) {
            const int t = lane + 64 * i;
            const int r = min(t, TB - 1) / H1, c = min(t, TB - 1) - r * H1;
            reg_dft<H2, -1>(v[i]);
            if (t < TB) {
#pragma unroll
                for (int d = 0; d < H2; ++d) buf[r * LP + c + H1 * d] = v[i][d];
            }
        }
        wave_lds_sync();
        // ---- even/odd split, frequencies m and H - m together: with
        // a = Z[m], b = conj(Z[H - m]) (Z[H] = Z[0]) and e = W^m (a - b),
        // W = exp(-2 pi i / N):  X[m] = (a + b)/2 - i e/2 and
        // X[H - m] = conj((a + b)/2 + i e/2).  Lane pairs m = lane + 64 i,
        // m <= H/2; words past H are zero ----
        {
            constexpr int NPI = (H / 2 + 1 + 63) / 64;   // pair iterations per row
            const float2 wl = root(lane, 0.5f / (float)H, -1.0f);   // W^lane
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const int64_t row = g * RW + r;
                const float2* z = buf + r * LP;
                uint32_t* out = xh + (row < nrows ? row : 0) * MP;
                static_for<0, NPI>([&](auto ii) {
                    constexpr int I = decltype(ii)::value;
                    const int m = lane + 64 * I;
                    if (m <= H / 2 && row < nrows) {
                        const float2 a = z[m];
                        const float2 bb = cconj(z[m == 0 ? 0 : H - m]);
                        const float2 e = cmul(rot_ct<2 * H, -1, 64 * I>(wl), csub(a, bb));
                        const float2 sm = cadd(a, bb);
                        // -i e = (e.y, -e.x)
                        out[m] = pack_bf16x2(0.5f * (sm.x + e.y), 0.5f * (sm.y - e.x));
                        if (m != 0 && 2 * m != H)
                            out[H - m] = pack_bf16x2(0.5f * (sm.x - e.y), -0.5f * (sm.y + e.x));
                        else if (m == 0)
                            out[H] = pack_bf16x2(0.5f * (sm.x - e.y), -0.5f * (sm.y + e.x));
                    }
                });
                if (lane < MP - H - 1 && row < nrows) out[H + 1 + lane] = 0u;
            }
        }
    }
}

// y_hat rows (MP bf16 pairs) -> y rows (N = 2 H) + bias, RW rows per wave and
// step.  Z[k] = (a + b)/2 + i W^-k (a - b)/2 with a = X[k], b = conj(X[H - k])
// (the imaginary parts of X[0] and X[H] dropped: a real row's spectrum has
// none), W = exp(-2 pi i / N); z[n] = sum_k Z[k] w_H^{-n k} by the same split
// (k = H2 a + b, n = c + H1 d); y[2n] = Re z[n] / H, y[2n+1] = Im z[n] / H.
// The merge fills Z in LDS (k and H - k together), step A reads it there,
// step B stores y (lanes c consecutive).  Workgroup g transforms rows
// g RW .. g RW + RW - 1.
template <int H1, int H2, int RW, typename TY>
__global__ __launch_bounds__(kRegThreads) void spec_irfft_reg(const uint32_t* __restrict__ yh,
                                                              TY* __restrict__ y,
                                                              const float* __restrict__ bias,
                                                              int Co, int nlat_out,
                                                              int64_t nrows) {
    constexpr int H = H1 * H2, N = 2 * H, MP = spec_mp_of(H);
    constexpr int P2 = H2 | 1, LP = H1 * P2;
    constexpr int TA = RW * H2, ITA = (TA + 63) / 64;
    constexpr int TB = RW * H1, ITB = (TB + 63) / 64;
    __shared__ float2 buf[RW * LP];
    const int lane = threadIdx.x;
    const int64_t g = blockIdx.x;   // the grid is the row-group count
    constexpr float sc = 1.0f / (float)H;

    // ---- merge, frequencies m and H - m together: with A = X[m],
    // B = conj(X[H - m]) (imaginary parts of X[0] and X[H] dropped),
    // s = A + B and e = W^-m (A - B):  Z[m] = (s + i e)/2 and
    // Z[H - m] = conj((s - i e)/2).  Z goes to LDS in natural order.
    {
        constexpr int NPI = (H / 2 + 1 + 63) / 64;   // pair iterations per row
        // every load first (addresses clamped to valid frequencies), so that
        // all are in flight together
        uint32_t la[RW][NPI], lb[RW][NPI];
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const uint32_t* src = yh + min(g * RW + r, nrows - 1) * MP;
#pragma unroll
            for (int I = 0; I < NPI; ++I) {
                const int m = min(lane + 64 * I, H / 2);
                la[r][I] = src[m];
                lb[r][I] = src[H - m];
            }
        }
        const float2 wl = root(lane, 1.0f / (float)N, 1.0f);   // W^-lane
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            float2* z = buf + r * LP;
            static_for<0, NPI>([&](auto ii) {
                constexpr int I = decltype(ii)::value;
                const int m = lane + 64 * I;
                if (m <= H / 2) {
                    float2 A = unpack_bf16x2(la[r][I]);
                    float2 Bc = cconj(unpack_bf16x2(lb[r][I]));
                    if (m == 0) {
                        A.y = 0.0f;
                        Bc.y = 0.0f;
                    }
                    const float2 e = cmul(rot_ct<N, 1, 64 * I>(wl), csub(A, Bc));
                    const float2 sm = cadd(A, Bc);
                    // i e = (-e.y, e.x)
                    z[m] = make_float2(0.5f * (sm.x - e.y), 0.5f * (sm.y + e.x));
                    if (m != 0 && 2 * m != H)
                        z[H - m] = make_float2(0.5f * (sm.x + e.y), 0.5f * (e.x - sm.y));
                }
            });
        }
    }
    wave_lds_sync();
    {
        // ---- step A: every lane reads its Z values, then the buffer is
        // rewritten in the exchange layout ----
        float2 va[ITA][H1];
#pragma unroll
        for (int i = 0; i < ITA; ++i) {
            const int t = min(lane + 64 * i, TA - 1);
            const int r = t / H2, b = t - r * H2;
#pragma unroll
            for (int a = 0; a < H1; ++a) va[i][a] = buf[r * LP + H2 * a + b];
        }
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < ITA; ++i) {
            const int t = lane + 64 * i;
            const int tc = min(t, TA - 1);
            const int r = tc / H2, b = tc - r * H2;
            reg_dft<H1, 1>(va[i]);
            const float2 w = root(b, 1.0f / (float)H, 1.0f);
            float2 p = w;
#pragma unroll
            for (int c = 1; c < H1; ++c) {
                va[i][c] = cmul(va[i][c], p);
                p = cmul(p, w);
            }
            if (t < TA) {
#pragma unroll
                for (int c = 0; c < H1; ++c) buf[r * LP + c * P2 + b] = va[i][c];
            }
        }
        wave_lds_sync();
        // ---- step B ----
        float2 v[ITB][H2];
#pragma unroll
        for (int i = 0; i < ITB; ++i) {
            const int t = min(lane + 64 * i, TB - 1);
            const int r = t / H1, c = t - r * H1;
#pragma unroll
            for (int b = 0; b < H2; ++b) v[i][b] = buf[r * LP + c * P2 + b];
        }
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < ITB; ++i) {
            const int t = lane + 64 * i;
            const int r = min(t, TB - 1) / H1, c = min(t, TB - 1) - r * H1;
            const int64_t row = g * RW + r;
            reg_dft<H2, 1>(v[i]);
            if (t < TB && row < nrows) {
                const float bv = bias ? bias[(row / nlat_out) % Co] : 0.0f;
                TY* out = y + row * N;
#pragma unroll
                for (int d = 0; d < H2; ++d) {
                    const int n = c + H1 * d;
                    const float2 o = make_float2(v[i][d].x * sc + bv, v[i][d].y * sc + bv);
                    if constexpr (sizeof(TY) == 4)
                        *reinterpret_cast<float2*>(out + 2 * n) = o;
                    else
                        *reinterpret_cast<uint32_t*>(out + 2 * n) = pack_bf16x2(o.x, o.y);
                }
            }
        }
    }
}

// w [Co][Ci][K] bf16 -> the GEMM's A operands in fragment order:
// wp[chunk][k-step][co / 32][lane][8], lane (l32, lg) holding row co = 32 * tile
// + l32 and pairs kappa = 16 k-step + 8 lg .. + 7 of the chunk, where a chunk's
// 256 pairs are ordered kappa = k * 32 + ci (basis index padded to 8 with
// zeros).  One wave's fragment is 1 KB of contiguous memory.
__global__ void spec_prep_w(const bf16_t* __restrict__ w, bf16_t* __restrict__ wp, int Co, int Ci,
                            int K) {
    const size_t n = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)Co * Ci * 8;
    if (n >= total) return;
    const int e = (int)(n & 7);
    const int lane = (int)((n >> 3) & 63);
    const size_t f = n >> 9;                  // (chunk * 16 + k-step) * (Co / 32) + tile
    const int tile = (int)(f % (Co / 32));
    const size_t cs = f / (Co / 32);
    const int ks = (int)(cs % 16), cc = (int)(cs / 16);
    const int co = tile * 32 + (lane & 31);
    const int kap = 16 * ks + 8 * (lane >> 5) + e;   // k * 32 + ci
    const int k = kap >> 5, ci = kap & 31;
    wp[n] = k < K ? w[((size_t)co * Ci + cc * 32 + ci) * K + k] : (bf16_t)0;
}

constexpr int kMt = 32;              // frequencies per work item (64 GEMM columns)
// B tile row of spec_mfma: pair (k, ci) at 40 k + ci (each 32-pair block padded by
// 8), 312 bf16 = 624 bytes per row (an odd multiple of 16 bytes).  The window
// sum's 8-byte writes (lanes differing in k) then fall into distinct banks, as
// do the GEMM's 16-byte reads (lanes differing in the row).
constexpr int kBts = 312;
constexpr int kBkb = 40;             // bf16 per k block of a tile row
constexpr int kSpecThreads = 256;
constexpr int kSpecMaxWin = 8;       // windows per output row (one 16-deep MFMA step)
constexpr int kXcds = 8;             // accelerator dies of the chip (L2 domains)

// Both sums of the forward equation for work items (batch b, output row j,
// 32 frequencies m0 ..), on the matrix cores, per 32-channel chunk.
//  * Window sum.  For one frequency, X_hat[ci, (k, re/im)] is the product of
//    x_hat[ci, (r, re/im)] (32 x 16: up to 8 windows) with the real 2 x 2
//    block form of conj(Psi_hat[k, r]) (16 x 32, columns (k, re/im), k < 8):
//    one v_mfma_f32_32x32x16_bf16.  The A operand is the bf16 (re, im) words
//    of x_hat as stored (lane = channel, four windows per lane half), read
//    from the chunk's spectra block in LDS, which is filled with coalesced
//    loads (eight lanes per 128-byte row); its 16-byte pieces are
//    XOR-swizzled by channel so that the lanes' reads hit distinct banks.
//    Each wave owns 8 of the 32 frequencies and builds their B operands at
//    the start of an item from the Psi_hat slice in LDS.  Results go to the
//    bf16 LDS tile bt[(m, re/im)][40 k + ci].
//  * Channel/basis GEMM: y_hat[co, (m, re/im)] += wp[co, (k, ci)] bt[(k, ci),
//    (m, re/im)], 4 waves, wave tile 32 x 64 (CO = 128) or 32 x 32 (CO = 64),
//    2 KT k-steps per chunk (the pairs of basis columns past KT are zero and
//    skipped), weights in fragment order.
// Persistent, in NX bands of the flattened output rows (b, j): workgroup g
// serves band g % NX (workgroups are dispatched to the XCDs round-robin, so a
// band stays on one XCD when NX is their count) and takes that band's items
// slot, slot + GX, ... (slot = g / NX, GX = gridDim.x / NX), where the band's
// items run tile-major: every row of the band for frequency tile 0, then tile
// 1, ...  The items in flight on an XCD then share their input rows' spectra
// in its L2.  A workgroup's (item, chunk) pairs form one stream, pipelined
// across item boundaries: once the window sum of position p has read its
// spectra, the block of p + 1 is loaded into the same LDS by DMA (its window
// rows fetched one position earlier) while p is computed, each weight
// fragment is reloaded for the next chunk right after its use (the weights
// do not depend on the item), and the next
// item's Psi_hat slice is loaded during the current item.
template <int CO, int KT>
__global__ __launch_bounds__(kSpecThreads) __attribute__((amdgpu_waves_per_eu(2))) void spec_mfma(
    const uint32_t* __restrict__ xh, const bf16_t* __restrict__ wp,
    const uint32_t* __restrict__ psih, const int32_t* __restrict__ win_ptr,
    const DevWindow* __restrict__ wins, bf16_t* __restrict__ yh, int B, int Ci, int nlat_in,
    int nlat_out, int MP, int NX, int64_t psih_zero, int nwmax) {
    __shared__ __attribute__((aligned(16))) bf16_t bt[64 * kBts];
    __shared__ __attribute__((aligned(16))) u32x4 xs[kSpecMaxWin * 32 * 8];   // [r][ci][piece]
    __shared__ __attribute__((aligned(16))) uint32_t ps[kSpecMaxWin * KT * kMt];
    __shared__ __attribute__((aligned(16))) bf16_t dump[32];   // 4 writes of 8 bytes, 8 apart
    constexpr int WGM = CO / 32;          // waves along the output channels
    constexpr int WGN = 4 / WGM;          // waves along the columns
    constexpr int NTW = 2 / WGN;          // 32-column MFMA tiles per wave

    const int ntiles = MP / kMt;
    const int GX = (int)gridDim.x / NX;   // workgroups per band (the grid is NX * GX)
    const int band = (int)blockIdx.x % NX, slot = (int)blockIdx.x / NX;
    const int nrows_all = B * nlat_out;
    const int r0 = (int)((int64_t)band * nrows_all / NX);
    const int brows = (int)((int64_t)(band + 1) * nrows_all / NX) - r0;
    // >= 1: slot < GX, and the host keeps GX <= (rows of the smallest band) * ntiles
    const int nmine = (brows * ntiles - slot + GX - 1) / GX;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int l32 = lane & 31, lg = lane >> 5;
    const int wm = wave % WGM, wn = wave / WGM;
    const int nchunks = Ci / 32;
    const int f0 = wave * 8;
    const size_t plane = (size_t)nlat_in * MP;

    // Item cursor: item n of this workgroup is l = slot + n GX of its band,
    // frequency tile mt = l / brows and band row ro = l % brows.  Cursors step
    // through the items in order (stopping at the last), so no item is decoded
    // by division more than once.
    struct Cur {
        int n, mt, ro;
    };
    auto cur_first = [&]() {
        Cur c;
        c.n = 0;
        c.mt = slot / brows;
        c.ro = slot - c.mt * brows;
        return c;
    };
    auto cur_next = [&](Cur& c) {
        if (c.n + 1 < nmine) {
            ++c.n;
            c.ro += GX;
            while (c.ro >= brows) {
                c.ro -= brows;
                ++c.mt;
            }
        }
    };
    auto cur_bj = [&](const Cur& c, int& b, int& j) {   // batch entry and output row
        j = r0 + c.ro;
        b = 0;
        if (B > 1) {
            b = j / nlat_out;
            j -= b * nlat_out;
        }
    };

    // ---- spectra stream: position p = (item p / nchunks, chunk p % nchunks).
    // The request cursor walks the positions in order (staying at the last).
    // A position's spectra block goes straight to LDS by DMA: wave w fills
    // windows 2w and 2w + 1.  LDS slot ((r * 32 + ci) * 8 + pos) holds the
    // 16-byte piece pos ^ (ci & 7) (4 frequencies) of channel ci's row in
    // window r.  Window slots past the row's windows repeat window 0 (valid,
    // finite; their B rows are zero).
    int lat_lo = 0, lat_hi = 0;     // input rows of windows 2w, 2w + 1 of the requested item
    int req_pos = 0, req_chunk = 0, req_b = 0;
    const int npos = nmine * nchunks;
    Cur rq = cur_first();
    auto request_item = [&]() {   // the window rows of the request cursor's item
        int j;
        cur_bj(rq, req_b, j);
        const int w0 = win_ptr[j], nw = win_ptr[j + 1] - w0;
        lat_lo = wins[w0 + (2 * wave < nw ? 2 * wave : 0)].lat;
        lat_hi = wins[w0 + (2 * wave + 1 < nw ? 2 * wave + 1 : 0)].lat;
    };
    auto request_next = [&]() {   // the next position
        if (req_pos + 1 < npos) {
            ++req_pos;
            if (++req_chunk == nchunks) {
                req_chunk = 0;
                cur_next(rq);
                request_item();
            }
        }
    };
    const uint32_t xs_lds =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void*)&xs[0]);
    // DMA of the requested position: 8 instructions per wave, instruction i
    // covering channels 8 (i % 4) .. + 7 of window 2w + i / 4 (64 slots)
    // this lane's source offsets (channel within the chunk and piece) of
    // instructions i and i + 4: constant over the stream
    size_t dma_off[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int ci = 8 * q + (lane >> 3);
        dma_off[q] = (size_t)ci * plane + 4 * ((lane & 7) ^ (ci & 7));
    }
    auto dma_x = [&]() {
        const size_t cb = (size_t)(req_b * Ci + req_chunk * 32) * plane + rq.mt * kMt;
        const uint32_t* blo = xh + cb + (size_t)uniform(lat_lo) * MP;
        const uint32_t* bhi = xh + cb + (size_t)uniform(lat_hi) * MP;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 2 * wave + (i >> 2);
            // window slots no output row has (r >= nwmax) are never read
            if (r < nwmax)
                dma_lds16((i < 4 ? blo : bhi) + dma_off[i & 3],
                          xs_lds + (uint32_t)((r * 32 + 8 * (i & 3)) * 8 * 16));
        }
    };

    // ---- Psi_hat slice of an item, ps[(r KT + k) kMt + ml], by DMA: KT
    // instructions of 64 16-byte slots (4 frequencies each), spread over the
    // waves; slots past the row's windows copy the table's zero block
    const uint32_t ps_lds =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void*)&ps[0]);
    auto dma_ps = [&](const Cur& c) {
        int b, j;
        cur_bj(c, b, j);
        const int w0 = win_ptr[j], nw = win_ptr[j + 1] - w0;
        for (int i = wave; i < KT; i += 4) {
            const int slot = 64 * i + lane;
            const int rk = slot >> 3, ml0 = (slot & 7) * 4;
            const uint32_t* src = rk < nw * KT
                                      ? psih + (size_t)(w0 * KT + rk) * MP + c.mt * kMt + ml0
                                      : psih + psih_zero;
            dma_lds16(src, ps_lds + (uint32_t)(i * 1024));
        }
    };

    Cur cur = cur_first();   // item n
    Cur nxt = cur;           // item n + 1 (the last item past the end)
    cur_next(nxt);
    dma_ps(cur);
    request_item();          // position 0
    dma_x();
    constexpr int NKS = 2 * KT;   // k-steps with non-zero basis columns
    u32x4 wq[NKS];
    // fragment (chunk, k-step) of this wave's 32 rows: wf[(chunk * 16 + k-step) * WGM * 64]
    const u32x4* wf = reinterpret_cast<const u32x4*>(wp) + wm * 64 + lane;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) wq[ks] = wf[(size_t)ks * WGM * 64];
    request_next();                    // rows of position 1
    wait_vmcnt<0>();
    __syncthreads();   // ps, zero columns, first spectra block

    for (int n = 0; n < nmine; ++n) {
        int b, j;
        cur_bj(cur, b, j);
        const int m0 = cur.mt * kMt;
        const int w0 = uniform(win_ptr[j]);
        const int nw = uniform(win_ptr[j + 1]) - w0;   // <= kSpecMaxWin (checked on the host)

        // B operands of the window sum: lane column n = 2 k + c (c: real,
        // imaginary part of X_hat), rows (r, re/im) for r = 4 lg .. 4 lg + 3
        // (windows past the row's are zero in ps; basis columns k >= KT are
        // never read by the GEMM, so their lanes take column KT - 1's values)
        u32x4 bq[8];
        {
            const int k = min(l32 >> 1, KT - 1), c = l32 & 1;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                // the wave's 8 frequencies of (window 4 lg + u, basis k): 32 bytes
                const u32x4* src =
                    reinterpret_cast<const u32x4*>(ps + ((4 * lg + u) * KT + k) * kMt + f0);
                const u32x4 lo = src[0], hi = src[1];
#pragma unroll
                for (int f = 0; f < 8; ++f) {
                    const uint32_t P = f < 4 ? lo[f] : hi[f - 4];   // bf16 (Pr, Pi), real low
                    // real column: (Pr, Pi); imaginary column: (-Pi, Pr)
                    bq[f][u] = c ? (__builtin_rotateleft32(P, 16) ^ 0x8000u) : P;
                }
            }
        }
        // A-operand reads: lane (channel l32, windows 4 lg + u, clamped to
        // window 0 past the row's windows), pieces 2 wave + h (swizzled by
        // the channel; 2 wave is even, so the h = 1 piece is the other's ^ 1)
        const int xsw = (2 * wave) ^ (l32 & 7);

        floatx16 acc[NTW];
#pragma unroll
        for (int t = 0; t < NTW; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;

        for (int cc = 0; cc < nchunks; ++cc) {
            // ---- window sum, one MFMA per frequency ----
            u32x4 xa[4][2];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = 4 * lg + u < nw ? 4 * lg + u : 0;
                    xa[u][h] = xs[(r * 32 + l32) * 8 + (xsw ^ h)];
                }
            wave_lds_sync();   // this wave's spectra reads are done
            __syncthreads();   // every wave's: the block may be overwritten
            // every wave has built its B operands from ps: the next item's
            // slice may replace it (completed with this position's DMA)
            if (cc == 0) dma_ps(nxt);
            dma_x();           // position p + 1 (the last position repeats at the end)
            request_next();    // rows of position p + 2
            // one MFMA per frequency, pipelined by one: the product of
            // frequency f + 1 is issued before frequency f's is converted and
            // written, so the matrix-core latency is hidden behind the writes
            auto window_mfma = [&](int f) {
                const u32x4 a = {xa[0][f >> 2][f & 3], xa[1][f >> 2][f & 3], xa[2][f >> 2][f & 3],
                                 xa[3][f >> 2][f & 3]};
                floatx16 d;
#pragma unroll
                for (int e = 0; e < 16; ++e) d[e] = 0.0f;
                return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                               __builtin_bit_cast(bf16x8_t, bq[f]), d,
                                                               0, 0, 0);
            };
            auto window_write = [&](const floatx16& d, int f) {
                // column (k, c) -> tile row 2 (f0 + f) + c, pairs (k, ci),
                // ci = 8 q + 4 lg + (0..3).  Columns KT <= k < 8 are written
                // but never read; lanes of columns k >= 8 (no tile block)
                // write the shared dump instead of branching around it.
                bf16_t* dst =
                    l32 < 16 ? bt + (2 * (f0 + f) + (l32 & 1)) * kBts + (l32 >> 1) * kBkb + 4 * lg
                             : dump;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint2 pk = make_uint2(pack_bf16x2(d[4 * q], d[4 * q + 1]),
                                                pack_bf16x2(d[4 * q + 2], d[4 * q + 3]));
                    *reinterpret_cast<uint2*>(dst + 8 * q) = pk;
                }
            };
            floatx16 dcur = window_mfma(0);
#pragma unroll
            for (int f = 0; f < 8; ++f) {
                floatx16 dnext;
                if (f + 1 < 8) dnext = window_mfma(f + 1);
                window_write(dcur, f);
                if (f + 1 < 8) dcur = dnext;
            }
            __syncthreads();   // tile complete
            // ---- channel/basis GEMM over this chunk's 256 (k, ci) pairs, at a
            // raised wave priority so that the SIMD keeps issuing its MFMAs
            // while the other workgroup's wave runs its window sum ----
            __builtin_amdgcn_s_setprio(2);
            const int cn = cc + 1 < nchunks ? cc + 1 : 0;   // weights of the next chunk
            const bf16_t* bb = bt + (wn * (64 / WGN) + l32) * kBts + 8 * lg;
            const u32x4* wnext = wf + (size_t)cn * 16 * WGM * 64;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8_t af = __builtin_bit_cast(bf16x8_t, wq[ks]);
#pragma unroll
                for (int t = 0; t < NTW; ++t) {
                    const bf16x8_t bf =
                        *reinterpret_cast<const bf16x8_t*>(bb + t * 32 * kBts +
                                                           (ks >> 1) * kBkb + 16 * (ks & 1));
                    // transposed product: lane column = output channel, rows =
                    // the tile's columns (frequency, re/im)
                    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf, af, acc[t], 0, 0, 0);
                }
                wq[ks] = wnext[(size_t)ks * WGM * 64];
                // reloads stay in k-step order right after their use: then the
                // next GEMM's wait for wq[0] leaves the newer spectra DMA in flight
                __builtin_amdgcn_sched_barrier(0);
            }
            // this wave's DMA of position p + 1 is complete; the NKS weight
            // reloads issued after it may stay in flight
            __builtin_amdgcn_s_setprio(0);
            wait_vmcnt<NKS>();
            __syncthreads();   // spectra of p + 1 in LDS; B tile free
        }
        // ---- y_hat (bf16 (re, im) pairs), staged through the free B tile so
        // that each store instruction writes whole 128-byte row segments.  The
        // lane holds channel co = 32 wm + l32 and columns 8 g + 4 lg + (0..3)
        // of its 32-column tile (g = e / 4); the staged tile is [co][64
        // columns] with rows of YS elements.  The next position's window sum
        // writes the B tile only after its first barrier, which every wave
        // reaches after its reads here. ----
        {
            constexpr int YS = 72;   // 144-byte rows: 16-byte aligned, spread over the banks
            static_assert(CO * YS <= 64 * kBts, "staged y_hat tile fits the B tile");
            const int co = wm * 32 + l32;
#pragma unroll
            for (int t = 0; t < NTW; ++t) {
                const int c0 = wn * (64 / WGN) + t * 32 + 4 * lg;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint2 pk = make_uint2(pack_bf16x2(acc[t][4 * g], acc[t][4 * g + 1]),
                                                pack_bf16x2(acc[t][4 * g + 2], acc[t][4 * g + 3]));
                    *reinterpret_cast<uint2*>(bt + co * YS + c0 + 8 * g) = pk;
                }
            }
            __syncthreads();   // staged tile complete
            // 16 bytes per lane: eight lanes per channel row of 64 columns
            bf16_t* ybase = yh + ((size_t)b * CO * nlat_out + j) * MP * 2 + 2 * m0;
#pragma unroll
            for (int it = 0; it < CO * 8 / kSpecThreads; ++it) {
                const int sl = tid + kSpecThreads * it;
                const int row = sl >> 3, pc = sl & 7;
                const u32x4 v = *reinterpret_cast<const u32x4*>(bt + row * YS + 8 * pc);
                *reinterpret_cast<u32x4*>(ybase + (size_t)row * nlat_out * MP * 2 + 8 * pc) = v;
            }
        }
        cur = nxt;
        cur_next(nxt);
    }
}

}  // namespace

// Which fused algorithm disco_fused_fwd takes for these arguments.
int fused_spectral_eligible(const disco_psi* psi, int x_dtype, int Ci, int Co, int groups) {
    const DevPsi& d = psi->dev;
    const HostPsi& h = psi->host;
    if (d.spec_mp <= 0 || x_dtype != DISCO_BF16 || groups != 1 || Ci % 32 != 0 ||
        (Co != 128 && Co != 64) || h.K > 8)
        return 0;
    if (d.max_windows > kSpecMaxWin) return 0;
    // DISCO_FUSED_PATH=toeplitz selects the direct matrix-core kernel instead
    const char* e = std::getenv("DISCO_FUSED_PATH");
    return e == nullptr || std::strcmp(e, "toeplitz") != 0;
}

int try_launch_fused_spectral(const disco_psi* psi, const void* x, const void* w,
                              const float* bias, void* y, int y_dtype, int B, int Ci, int Co,
                              int groups, hipStream_t st, int* rc) {
    if (!fused_spectral_eligible(psi, DISCO_BF16, Ci, Co, groups) || B <= 0) return 0;
    const DevPsi& d = psi->dev;
    const HostPsi& h = psi->host;
    const disco_psi_desc& D = h.desc;
    const int N = D.nlon_in, H = N / 2, MP = d.spec_mp, K = h.K;
    SpecPlan pl;
    pl.n = d.spec_nrad;
    for (int i = 0; i < kSpecMaxRadix; ++i) pl.r[i] = d.spec_radix[i];

    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t xh_bytes = up((size_t)B * Ci * D.nlat_in * MP * 4);
    const size_t yh_bytes = up((size_t)B * Co * D.nlat_out * MP * 4);
    const size_t wp_bytes = up((size_t)Co * Ci * 8 * 2);
    void* ws = nullptr;
    hipError_t e = hipMallocAsync(&ws, xh_bytes + yh_bytes + wp_bytes, st);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        *rc = set_error(e == hipErrorOutOfMemory ? DISCO_ENOMEM : DISCO_EHIP,
                        "hipMallocAsync for the spectral workspace failed: %s",
                        hipGetErrorString(e));
        return 1;
    }
    uint32_t* xh = static_cast<uint32_t*>(ws);
    bf16_t* yh = reinterpret_cast<bf16_t*>(static_cast<char*>(ws) + xh_bytes);
    bf16_t* wpd = reinterpret_cast<bf16_t*>(static_cast<char*>(ws) + xh_bytes + yh_bytes);
    const uint32_t* psih = static_cast<const uint32_t*>(d.spec_psih);

    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    (void)hipGetLastError();
    // the register-resident transforms cover these half lengths (their MP is
    // the table's)
    const bool reg = (H == 720 || H == 360 || H == 180) && MP == spec_mp_of(H);
    // one-wave workgroups, one group of rw rows each
    auto reg_grid = [](int64_t rows, int rw) { return dim3((unsigned)((rows + rw - 1) / rw)); };

    const size_t nwp = (size_t)Co * Ci * 8;
    {
        KernelTimer timer("spec_prep_w", st);
        hipLaunchKernelGGL(spec_prep_w, dim3((unsigned)((nwp + 255) / 256)), dim3(256), 0, st,
                           static_cast<const bf16_t*>(w), wpd, Co, Ci, K);
    }
    const size_t fft_lds = (size_t)(kFftRows + 1) * H * sizeof(float2);
    const int64_t xrows = (int64_t)B * Ci * D.nlat_in;
    const uint32_t* x32 = static_cast<const uint32_t*>(x);
#define DISCO_RF(H1, H2, RW)                                                                   \
    hipLaunchKernelGGL((spec_rfft_reg<H1, H2, RW>),                                            \
                       reg_grid(xrows, RW),                                                    \
                       dim3(kRegThreads), 0, st, x32, xh, xrows)
    {
    KernelTimer timer("spec_rfft", st);
    if (reg && H == 720) {
        DISCO_RF(16, 45, 4);
    } else if (reg && H == 360) {
        DISCO_RF(8, 45, 8);
    } else if (reg && H == 180) {
        DISCO_RF(4, 45, 16);
    } else {
        hipLaunchKernelGGL(spec_rfft, dim3((unsigned)((xrows + kFftRows - 1) / kFftRows)),
                           dim3(kFftThreads), fft_lds, st, static_cast<const bf16_t*>(x), xh, N,
                           MP, xrows, pl);
    }
    }
#undef DISCO_RF
    // bands of output rows, one per XCD; GX workgroups per band, at most the
    // smallest band's item count
    const int64_t nrows_all = (int64_t)B * D.nlat_out;
    const int NX = (int)std::min<int64_t>(kXcds, nrows_all);
    const int64_t min_items = nrows_all / NX * (MP / kMt);
    const int GX = (int)std::max<int64_t>(1, std::min<int64_t>(min_items, 2 * (int64_t)ncu / NX));
    dim3 grid((unsigned)(NX * GX));
#define DISCO_SM(CC, KK)                                                                     \
    hipLaunchKernelGGL((spec_mfma<CC, KK>), grid, dim3(kSpecThreads), 0, st, xh, wpd,         \
                       psih, d.win_ptr, d.windows, yh, B, Ci, D.nlat_in, D.nlat_out, MP, NX, \
                       (int64_t)h.windows.size() * K * MP, (int)d.max_windows)
#define DISCO_SM_K(CC)                                                                       \
    switch (K) {                                                                             \
        case 1: DISCO_SM(CC, 1); break;                                                      \
        case 2: DISCO_SM(CC, 2); break;                                                      \
        case 3: DISCO_SM(CC, 3); break;                                                      \
        case 4: DISCO_SM(CC, 4); break;                                                      \
        case 5: DISCO_SM(CC, 5); break;                                                      \
        case 6: DISCO_SM(CC, 6); break;                                                      \
        case 7: DISCO_SM(CC, 7); break;                                                      \
        default: DISCO_SM(CC, 8); break;                                                     \
    }
    {
        KernelTimer timer("spec_mfma", st);
        if (Co == 128) {
            DISCO_SM_K(128)
        } else {
            DISCO_SM_K(64)
        }
    }
#undef DISCO_SM_K
#undef DISCO_SM
    const int64_t yrows = (int64_t)B * Co * D.nlat_out;
    const dim3 igrid((unsigned)((yrows + kFftRows - 1) / kFftRows));
    const uint32_t* yh32 = reinterpret_cast<const uint32_t*>(yh);
#define DISCO_IR(H1, H2, RW, TY)                                                               \
    hipLaunchKernelGGL((spec_irfft_reg<H1, H2, RW, TY>),                                       \
                       reg_grid(yrows, RW),                                                    \
                       dim3(kRegThreads), 0, st, yh32, static_cast<TY*>(y), bias, Co,          \
                       D.nlat_out, yrows)
#define DISCO_IR_T(H1, H2, RW)                 \
    if (y_dtype == DISCO_F32) {                \
        DISCO_IR(H1, H2, RW, float);           \
    } else {                                   \
        DISCO_IR(H1, H2, RW, bf16_t);          \
    }
    {
    KernelTimer timer("spec_irfft", st);
    if (reg && H == 720) {
        DISCO_IR_T(16, 45, 4)
    } else if (reg && H == 360) {
        DISCO_IR_T(8, 45, 8)
    } else if (reg && H == 180) {
        DISCO_IR_T(4, 45, 16)
    } else if (y_dtype == DISCO_F32)
        hipLaunchKernelGGL(spec_irfft<float>, igrid, dim3(kFftThreads), fft_lds, st,
                           reinterpret_cast<const uint32_t*>(yh), static_cast<float*>(y), bias, N,
                           MP, Co, D.nlat_out, yrows, pl);
    else
        hipLaunchKernelGGL(spec_irfft<bf16_t>, igrid, dim3(kFftThreads), fft_lds, st,
                           reinterpret_cast<const uint32_t*>(yh), static_cast<bf16_t*>(y), bias, N,
                           MP, Co, D.nlat_out, yrows, pl);
    }
#undef DISCO_IR_T
#undef DISCO_IR
    hipError_t le = hipGetLastError();
    hipError_t fe = hipFreeAsync(ws, st);
    if (le != hipSuccess) {
        *rc = set_error(DISCO_EHIP, "spectral fused launch failed: %s", hipGetErrorString(le));
        return 1;
    }
    if (fe != hipSuccess) {
        (void)hipGetLastError();
        *rc = set_error(DISCO_EHIP, "hipFreeAsync failed: %s", hipGetErrorString(fe));
        return 1;
    }
    *rc = DISCO_OK;
    return 1;
}

}  // namespace disco
