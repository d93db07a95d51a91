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
#include "spectral_dft.h"

namespace disco {

namespace {

using namespace specdft;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct SpecPlan {
    int32_t n;
    int32_t r[kSpecMaxRadix];
};

// complex arithmetic, short butterflies and the register DFTs: spectral_dft.h
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

__device__ __forceinline__ void spec_store(uint32_t* p, int64_t i, float2 v) {
    p[i] = pack_bf16x2(v.x, v.y);
}

constexpr int kFftThreads = 256;
constexpr int kFftRows = kFftThreads / 64;   // one wave per row

// Twiddle table of the workgroup: twl[e] = exp(-2 pi i e / H), e < H.
__device__ __forceinline__ void fill_twiddles(float2* twl, int H) {
    const float inv_h = 1.0f / (float)H;
    for (int e = threadIdx.x; e < H; e += blockDim.x) twl[e] = root(e, inv_h, -1.0f);
}

// Spectrum storage: bf16 (re, im) pairs in one 32-bit word (real part low),
// or float32 pairs.
__device__ __forceinline__ float2 spec_load(const uint32_t* p, int64_t i) {
    const uint32_t v = p[i];
    return make_float2(__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u));
}
__device__ __forceinline__ float2 spec_load(const float2* p, int64_t i) { return p[i]; }
__device__ __forceinline__ void spec_store(float2* p, int64_t i, float2 v) { p[i] = v; }
// two consecutive samples of a real row
__device__ __forceinline__ float2 sample_pair(const bf16_t* row, int n) {
    const uint32_t v = reinterpret_cast<const uint32_t*>(row)[n];
    return make_float2(__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u));
}
__device__ __forceinline__ float2 sample_pair(const float* row, int n) {
    return reinterpret_cast<const float2*>(row)[n];
}

// x rows (N real, bf16 or float32) -> x_hat rows (MP spectrum words;
// frequencies past N/2 are zero).  One wave per row, four rows per workgroup;
// LDS: one H-point buffer per row and the H-point twiddle table.  Waves past
// the last row leave after the table is built.
template <typename TX, typename TS>
__global__ __launch_bounds__(kFftThreads) void spec_rfft(const TX* __restrict__ x,
                                                         TS* __restrict__ xh, int N, int MP,
                                                         int64_t nrows, SpecPlan pl) {
    extern __shared__ float2 sm[];
    const int H = N / 2;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kFftRows + wave;
    const bool live = row < nrows;
    float2* b0 = sm + (size_t)wave * H;
    float2* twl = sm + (size_t)kFftRows * H;
    fill_twiddles(twl, H);
    const TX* xr = x + (live ? row : 0) * (size_t)N;
    for (int n = lane; n < H; n += 64) b0[n] = sample_pair(xr, n);   // samples 2n, 2n + 1
    __syncthreads();   // the twiddle table
    if (!live) return;
    fft_wave(b0, H, pl, twl, -1.0f, lane);
    const float2* z = b0;
    // X[m] = (a + b)/2 - i W^m (a - b)/2, a = Z[m mod H], b = conj(Z[(H - m) mod H]),
    // W = exp(-2 pi i / N)
    TS* out = xh + row * (size_t)MP;
    const float inv_n = 0.5f / (float)H;
    for (int m = lane; m < MP; m += 64) {
        float2 X = make_float2(0.0f, 0.0f);
        if (m <= H) {
            const float2 a = z[m == H ? 0 : m];
            const float2 b = cconj(z[m == 0 ? 0 : H - m]);
            const float2 e = cmul(root(m, inv_n, -1.0f), csub(a, b));
            X = cadd(cscale(cadd(a, b), 0.5f), cscale(make_float2(e.y, -e.x), 0.5f));
        }
        spec_store(out, m, X);
    }
}

// y_hat rows (MP bf16 pairs, frequencies 0..N/2 used) -> y rows (N) + bias,
// one wave per row (LDS as for spec_rfft).  The imaginary parts of the zero and N/2 frequencies are
// dropped (a real row's spectrum has none).
template <typename TS, typename TY>
__global__ __launch_bounds__(kFftThreads) void spec_irfft(const TS* __restrict__ yh,
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
    const TS* src = yh + (live ? row : 0) * (size_t)MP;
    auto spec = [&](int m) { return spec_load(src, m); };
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

__device__ __forceinline__ float2 unpack_bf16x2(uint32_t v) {
    return make_float2(__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u));
}

constexpr int kRegThreads = 64;   // one wave per workgroup

constexpr int spec_mp_of(int H) { return (H + 32) / 32 * 32; }   // (H + 1) rounded up to 32

// w [Co][Ci][K] bf16 -> the GEMM's A operands in fragment order:
// wp[chunk][k-step][co / 32][lane][8], lane (l32, lg) holding row co = 32 * tile
// + l32 and pairs kappa = 16 k-step + 8 lg .. + 7 of the chunk, where a chunk's
// 256 pairs are ordered kappa = k * 32 + ci (basis index padded to 8 with
// zeros).  One wave's fragment is 1 KB of contiguous memory.
__device__ __forceinline__ void prep_w_elem(const bf16_t* __restrict__ w, bf16_t* __restrict__ wp,
                                            int Co, int Ci, int K, size_t n, int wt) {
    const int e = (int)(n & 7);
    const int lane = (int)((n >> 3) & 63);
    const size_t f = n >> 9;                  // (chunk * 16 + k-step) * (Co / 32) + tile
    const int tile = (int)(f % (Co / 32));
    const size_t cs = f / (Co / 32);
    const int ks = (int)(cs % 16), cc = (int)(cs / 16);
    const int co = tile * 32 + (lane & 31);
    const int kap = 16 * ks + 8 * (lane >> 5) + e;   // k * 32 + ci
    const int k = kap >> 5, ci = kap & 31;
    // wt: w is stored [Ci][Co][K] (the forward layer's weights, read by the
    // adjoint, whose GEMM maps the layer's output channels to its inputs)
    const size_t src = wt ? ((size_t)(cc * 32 + ci) * Co + co) * K + k
                          : ((size_t)co * Ci + cc * 32 + ci) * K + k;
    wp[n] = k < K ? w[src] : (bf16_t)0;
}

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
// and is slower.)  The first nprep workgroups instead write the weight
// fragments (kPrepPerWg elements each, the work of spec_prep_w), so that the
// call needs no launch of its own for them.
constexpr int kPrepPerWg = 64 * 16;
template <int H1, int H2, int RW>
__global__ __launch_bounds__(kRegThreads) void spec_rfft_reg(const uint32_t* __restrict__ x,
                                                             uint32_t* __restrict__ xh,
                                                             int64_t nrows,
                                                             const bf16_t* __restrict__ w,
                                                             bf16_t* __restrict__ wp, int Co,
                                                             int Ci, int K, int nprep, int wt) {
    constexpr int H = H1 * H2, MP = spec_mp_of(H);
    constexpr int P2 = H2 | 1, LP = H1 * P2;
    constexpr int TA = RW * H2, ITA = (TA + 63) / 64;
    constexpr int TB = RW * H1, ITB = (TB + 63) / 64;
    static_assert(LP >= H, "the split needs H entries per row");
    static_assert(MP - H - 1 <= 64, "one lane per padding word");
    __shared__ float2 buf[RW * LP];
    const int lane = threadIdx.x;
    if ((int)blockIdx.x < nprep) {
        const size_t total = (size_t)Co * Ci * 8;
        const size_t n0 = (size_t)blockIdx.x * kPrepPerWg + lane;
#pragma unroll 4
        for (int t = 0; t < kPrepPerWg / 64; ++t) {
            const size_t n = n0 + 64 * t;
            if (n < total) prep_w_elem(w, wp, Co, Ci, K, n, wt);
        }
        return;
    }
    const int64_t g = (int64_t)blockIdx.x - nprep;   // the grid is nprep + the row-group count

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
//
// FOLD = 2 (longitude stride 2): the rows of yh are the spectra Y of the
// stride-1 correlation at 2N points (frequencies 0 .. N, row stride mp_in),
// and the output keeps every second longitude.  Decimating by two sums the
// two aliases of each frequency: X[m] = (Y[m] + conj(Y[N - m])) / 2.
template <int H1, int H2, int RW, typename TY, int FOLD>
__global__ __launch_bounds__(kRegThreads) void spec_irfft_reg(const uint32_t* __restrict__ yh,
                                                              TY* __restrict__ y,
                                                              const float* __restrict__ bias,
                                                              int Co, int nlat_out,
                                                              int64_t nrows, int mp_in) {
    constexpr int H = H1 * H2, N = 2 * H;
    static_assert(FOLD == 1 || FOLD == 2, "longitude strides 1 and 2");
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
        uint32_t fa[FOLD == 2 ? RW : 1][FOLD == 2 ? NPI : 1];   // aliases (stride 2)
        uint32_t fb[FOLD == 2 ? RW : 1][FOLD == 2 ? NPI : 1];
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const uint32_t* src = yh + min(g * RW + r, nrows - 1) * (int64_t)mp_in;
#pragma unroll
            for (int I = 0; I < NPI; ++I) {
                const int m = min(lane + 64 * I, H / 2);
                la[r][I] = src[m];
                lb[r][I] = src[H - m];
                if constexpr (FOLD == 2) {
                    fa[r][I] = src[N - m];
                    fb[r][I] = src[H + m];
                }
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
                    if constexpr (FOLD == 2) {
                        // X[m] = (Y[m] + conj(Y[N - m]))/2, and X[H - m] with
                        // conj(Y[N - (H - m)]) = conj(Y[H + m])
                        A = cscale(cadd(A, cconj(unpack_bf16x2(fa[r][I]))), 0.5f);
                        Bc = cscale(cadd(Bc, unpack_bf16x2(fb[r][I])), 0.5f);
                    }
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

// bf16 samples -> 32-bit words (sample, 0): rows of n samples become rows of
// 2 n samples with a zero after each (the adjoint of keeping every second
// longitude)
__global__ void spec_zero_insert(const bf16_t* __restrict__ in, uint32_t* __restrict__ out,
                                 size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = (uint32_t)__builtin_bit_cast(uint16_t, in[i]);
}

// the weight fragments alone (for the Stockham transforms' launches)
__global__ void spec_prep_w(const bf16_t* __restrict__ w, bf16_t* __restrict__ wp, int Co, int Ci,
                            int K, int wt) {
    const size_t n = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n < (size_t)Co * Ci * 8) prep_w_elem(w, wp, Co, Ci, K, n, wt);
}

constexpr int kMt = 32;              // frequencies per work item (64 GEMM columns)
// B tile row r of spec_mfma: pair (k, ci) at 40 (k ^ ((r >> 1) & 7)) + ci (32-pair
// blocks padded by 8, their order permuted by the row pair), 320 bf16 = 640
// bytes per row (160 words: 4 times an odd number).  On the 64-bank LDS the
// GEMM's 16-byte reads (16 lanes of consecutive rows per phase) then cover
// all banks, and so do the window sum's 8-byte writes (32 lanes per phase:
// 8 basis blocks of two rows, in 2 x 4 lanes).
constexpr int kBts = 320;
constexpr int kBkb = 40;             // bf16 per k block of a tile row
constexpr int kSpecThreads = 256;
constexpr int kSpecMaxWin = 16;      // windows per output row: one or two 16-deep MFMA steps
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
//    XOR-swizzled by channel pair, so that the 16 lanes of a read phase (two
//    channels per 256 bytes of banks) hit distinct banks.
//    Each wave owns 8 of the 32 frequencies and builds their B operands at
//    the start of an item from the Psi_hat slice in LDS.  Results go to the
//    bf16 LDS tile bt[(m, re/im)][40 (k ^ (m & 7)) + ci].
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
// NW (8 or 16) is the window capacity: the window sum is one 16-deep MFMA
// step per 8 windows (rows with at most 8 windows skip the second step).
// With NW = 8 two workgroups fit a compute unit; NW = 16 doubles the spectra
// and Psi_hat blocks and takes the whole LDS.
template <int CO, int KT, int NW>
__global__ __launch_bounds__(kSpecThreads) __attribute__((amdgpu_waves_per_eu(NW == 8 ? 2 : 1))) void spec_mfma(
    const uint32_t* __restrict__ xh, const bf16_t* __restrict__ wp,
    const uint32_t* __restrict__ psih, const int32_t* __restrict__ win_ptr,
    const DevWindow* __restrict__ wins, bf16_t* __restrict__ yh, int B, int Ci, int nlat_in,
    int nlat_out, int MP, int NX, int64_t psih_zero, int nwmax, int NP) {
    static_assert(NW == 8 || NW == 16, "window capacity");
    constexpr int NS = NW / 8;            // window-sum MFMA steps
    constexpr int WPW = NW / 4;           // windows whose spectra each wave copies
    __shared__ __attribute__((aligned(16))) bf16_t bt[64 * kBts];
    __shared__ __attribute__((aligned(16))) u32x4 xs[NW * 32 * 8];   // [r][ci][piece]
    __shared__ __attribute__((aligned(16))) uint32_t ps[NW * KT * kMt];
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
    // frequency tile mt = l / brows and band row ro = l % brows.  With NP = 2
    // an item is visited twice, once per half of its row's windows (part 0:
    // the first ceil(nw / 2), part 1: the rest; the host passes NP = 2 only
    // when every row has at least two windows), and the channel/basis GEMM
    // accumulates both halves before y_hat is stored.  Cursors step through
    // the (item, part) pairs in order (stopping at the last), so no item is
    // decoded by division more than once.
    struct Cur {
        int n, mt, ro, part;
    };
    auto cur_first = [&]() {
        Cur c;
        c.n = 0;
        c.mt = slot / brows;
        c.ro = slot - c.mt * brows;
        c.part = 0;
        return c;
    };
    auto cur_next = [&](Cur& c) {
        if (c.part + 1 < NP) {
            ++c.part;
        } else if (c.n + 1 < nmine) {
            c.part = 0;
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
    // the windows of the cursor's (item, part): [w0, w0 + nw)
    auto cur_windows = [&](const Cur& c, int j, int& w0, int& nw) {
        w0 = win_ptr[j];
        nw = win_ptr[j + 1] - w0;
        if (NP == 2) {
            const int h = (nw + 1) >> 1;
            if (c.part == 0) {
                nw = h;
            } else {
                w0 += h;
                nw -= h;
            }
        }
    };

    // ---- spectra stream: position p = (item p / nchunks, chunk p % nchunks).
    // The request cursor walks the positions in order (staying at the last).
    // A position's spectra block goes straight to LDS by DMA: wave w fills
    // windows WPW w .. WPW w + WPW - 1.  LDS slot ((r * 32 + ci) * 8 + pos)
    // holds the 16-byte piece pos ^ ((ci >> 1) & 7) (4 frequencies) of channel ci's
    // row in window r.  Window slots past the row's windows repeat window 0
    // (valid, finite; their B rows are zero).
    int lat_w[WPW];                 // input rows of this wave's windows of the requested item
    int req_pos = 0, req_chunk = 0, req_b = 0;
    const int npos = nmine * NP * nchunks;
    Cur rq = cur_first();
    auto request_item = [&]() {   // the window rows of the request cursor's item
        int j, w0, nw;
        cur_bj(rq, req_b, j);
        cur_windows(rq, j, w0, nw);
#pragma unroll
        for (int u = 0; u < WPW; ++u) {
            const int r = WPW * wave + u;
            lat_w[u] = wins[w0 + (r < nw ? r : 0)].lat;
        }
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
    // DMA of the requested position: 4 WPW instructions per wave, instruction
    // i covering channels 8 (i % 4) .. + 7 of window WPW w + i / 4 (64 slots)
    // this lane's source offsets (channel within the chunk and piece) of
    // instructions i and i + 4: constant over the stream
    size_t dma_off[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int ci = 8 * q + (lane >> 3);
        dma_off[q] = (size_t)ci * plane + 4 * ((lane & 7) ^ ((ci >> 1) & 7));
    }
    auto dma_x = [&]() {
        const size_t cb = (size_t)(req_b * Ci + req_chunk * 32) * plane + rq.mt * kMt;
#pragma unroll
        for (int u = 0; u < WPW; ++u) {
            const int r = WPW * wave + u;
            const uint32_t* src = xh + cb + (size_t)uniform(lat_w[u]) * MP;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // window slots no output row has (r >= nwmax) are never read
                if (r < nwmax)
                    dma_lds16(src + dma_off[q], xs_lds + (uint32_t)((r * 32 + 8 * q) * 8 * 16));
            }
        }
    };

    // ---- Psi_hat slice of an item, ps[(r KT + k) kMt + ml], by DMA: NS KT
    // instructions of 64 16-byte slots (4 frequencies each), spread over the
    // waves; slots past the row's windows copy the table's zero block
    const uint32_t ps_lds =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void*)&ps[0]);
    auto dma_ps = [&](const Cur& c) {
        int b, j, w0, nw;
        cur_bj(c, b, j);
        cur_windows(c, j, w0, nw);
        for (int i = wave; i < NS * KT; i += 4) {
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

    floatx16 acc[NTW];   // y_hat of the current item, over its NP parts
    for (int v = 0; v < nmine * NP; ++v) {
        int b, j, w0, nw;
        cur_bj(cur, b, j);
        const int m0 = cur.mt * kMt;
        cur_windows(cur, j, w0, nw);
        nw = uniform(nw);   // <= kSpecMaxWin (checked on the host)

        // B operands of the window sum: lane column n = 2 k + c (c: real,
        // imaginary part of X_hat), rows (r, re/im) for r = 4 lg .. 4 lg + 3
        // (windows past the row's are zero in ps; basis columns k >= KT are
        // never read by the GEMM, so their lanes take column KT - 1's values)
        // step st covers windows 8 st .. 8 st + 7; rows with at most 8
        // windows skip the second step (uniform)
        const bool two = NS == 2 && nw > 8;
        u32x4 bq[NS][8];
        {
            const int k = min(l32 >> 1, KT - 1), c = l32 & 1;
#pragma unroll
            for (int st = 0; st < NS; ++st)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                // the wave's 8 frequencies of (window 8 st + 4 lg + u, basis k): 32 bytes
                const u32x4* src = reinterpret_cast<const u32x4*>(
                    ps + ((8 * st + 4 * lg + u) * KT + k) * kMt + f0);
                const u32x4 lo = src[0], hi = src[1];
#pragma unroll
                for (int f = 0; f < 8; ++f) {
                    const uint32_t P = f < 4 ? lo[f] : hi[f - 4];   // bf16 (Pr, Pi), real low
                    // real column: (Pr, Pi); imaginary column: (-Pi, Pr)
                    bq[st][f][u] = c ? (__builtin_rotateleft32(P, 16) ^ 0x8000u) : P;
                }
            }
        }
        // A-operand reads: lane (channel l32, windows 4 lg + u, clamped to
        // window 0 past the row's windows), pieces 2 wave + h (swizzled by
        // the channel; 2 wave is even, so the h = 1 piece is the other's ^ 1)
        const int xsw = (2 * wave) ^ ((l32 >> 1) & 7);

        if (cur.part == 0) {
#pragma unroll
            for (int t = 0; t < NTW; ++t)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;
        }

        for (int cc = 0; cc < nchunks; ++cc) {
            // ---- window sum, one MFMA per frequency ----
            u32x4 xa[NS][4][2];
#pragma unroll
            for (int st = 0; st < NS; ++st)
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = 8 * st + 4 * lg + u < nw ? 8 * st + 4 * lg + u : 0;
                    xa[st][u][h] = xs[(r * 32 + l32) * 8 + (xsw ^ h)];
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
                floatx16 d;
#pragma unroll
                for (int e = 0; e < 16; ++e) d[e] = 0.0f;
                const u32x4 a = {xa[0][0][f >> 2][f & 3], xa[0][1][f >> 2][f & 3],
                                 xa[0][2][f >> 2][f & 3], xa[0][3][f >> 2][f & 3]};
                d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                            __builtin_bit_cast(bf16x8_t, bq[0][f]),
                                                            d, 0, 0, 0);
                if constexpr (NS == 2) {
                    if (two) {
                        const u32x4 a1 = {xa[NS - 1][0][f >> 2][f & 3], xa[NS - 1][1][f >> 2][f & 3],
                                          xa[NS - 1][2][f >> 2][f & 3], xa[NS - 1][3][f >> 2][f & 3]};
                        d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8_t, a1),
                            __builtin_bit_cast(bf16x8_t, bq[NS - 1][f]), d, 0, 0, 0);
                    }
                }
                return d;
            };
            auto window_write = [&](const floatx16& d, int f) {
                // column (k, c) -> tile row 2 (f0 + f) + c, pairs (k, ci),
                // ci = 8 q + 4 lg + (0..3), in block k ^ f of the row ((row >>
                // 1) & 7 = f: f0 is a multiple of 8).  Columns KT <= k < 8
                // are written but never read; lanes of columns k >= 8 have no
                // tile block and write nothing.
                if (l32 < 16) {
                    bf16_t* dst = bt + (2 * (f0 + f) + (l32 & 1)) * kBts +
                                  ((l32 >> 1) ^ f) * kBkb + 4 * lg;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint2 pk = make_uint2(pack_bf16x2(d[4 * q], d[4 * q + 1]),
                                                    pack_bf16x2(d[4 * q + 2], d[4 * q + 3]));
                        *reinterpret_cast<uint2*>(dst + 8 * q) = pk;
                    }
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
            // block permutation of this lane's rows (wn * (64 / WGN) + 32 t +
            // l32: the same for every t)
            const int bsw = (l32 >> 1) & 7;
            const u32x4* wnext = wf + (size_t)cn * 16 * WGM * 64;
            auto bfrag = [&](int ks, int t) {
                return *reinterpret_cast<const bf16x8_t*>(bb + t * 32 * kBts +
                                                          ((ks >> 1) ^ bsw) * kBkb +
                                                          16 * (ks & 1));
            };
            // B fragments read two k-steps ahead of their MFMAs, so that the
            // LDS latency hides behind the two steps in between
            bf16x8_t bq0[NTW], bq1[NTW];
#pragma unroll
            for (int t = 0; t < NTW; ++t) bq0[t] = bfrag(0, t);
#pragma unroll
            for (int t = 0; t < NTW; ++t) bq1[t] = bfrag(1, t);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8_t af = __builtin_bit_cast(bf16x8_t, wq[ks]);
                bf16x8_t bn[NTW];
                if (ks + 2 < NKS) {
#pragma unroll
                    for (int t = 0; t < NTW; ++t) bn[t] = bfrag(ks + 2, t);
                }
                // transposed product: lane column = output channel, rows = the
                // tile's columns (frequency, re/im)
#pragma unroll
                for (int t = 0; t < NTW; ++t)
                    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bq0[t], af, acc[t], 0, 0, 0);
#pragma unroll
                for (int t = 0; t < NTW; ++t) {
                    bq0[t] = bq1[t];
                    if (ks + 2 < NKS) bq1[t] = bn[t];
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
        if (cur.part + 1 < NP) {   // the item's other half of its windows next
            cur = nxt;
            cur_next(nxt);
            continue;
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

// ---------------------------------------------------------------------------
// Float32 layers (stride 1): both sums per frequency on the vector ALUs, in
// float32, on float32 spectra (Psi_hat tabulated in float64 and rounded once
// to float32).  One workgroup per item (batch b, output row j, 32
// frequencies m0 ..); input channels in chunks of 8:
//   X_hat[ci, k, m] = sum_windows x_hat[b, ci, i, m] conj(Psi_hat[k, window, m])
//     into an LDS tile, thread (ci, m);
//   y_hat[co, m] += sum_{ci, k} w[co, ci, k] X_hat[ci, k, m]
//     thread (co = cl + 32 r, m = 4 q .. 4 q + 3), the chunk's weights staged
//     in LDS (one word per (co, ci, k), read by the 8 lanes of one co).
// ---------------------------------------------------------------------------
constexpr int kS32M = 32;    // frequencies per item
constexpr int kS32C = 8;     // input channels per chunk
template <int KT, int COR>
__global__ __launch_bounds__(kSpecThreads) void spec32_conv(
    const float2* __restrict__ xh, const float* __restrict__ w, const float2* __restrict__ psih,
    const int32_t* __restrict__ win_ptr, const DevWindow* __restrict__ wins,
    float2* __restrict__ yh, int Ci, int Co, int nlat_in, int nlat_out, int MP, int nwmax,
    int wtr) {
    extern __shared__ float2 s32[];
    float2* ps = s32;                                  // [nwmax][KT][32]
    float2* xt = ps + (size_t)nwmax * KT * kS32M;      // [kS32C][KT][32]
    float* wt = reinterpret_cast<float*>(xt + kS32C * KT * kS32M);   // [Co][kS32C][KT]
    int* lat = reinterpret_cast<int*>(wt + (size_t)Co * kS32C * KT); // [nwmax]
    const int tid = threadIdx.x;
    const int ntile = MP / kS32M;
    int item = blockIdx.x;
    const int mt = item % ntile;
    item /= ntile;
    const int j = item % nlat_out, b = item / nlat_out;
    const int m0 = mt * kS32M;
    const int w0 = win_ptr[j], nw = win_ptr[j + 1] - w0;   // <= nwmax
    for (int e = tid; e < nw * KT * kS32M; e += kSpecThreads) {
        const int m = e % kS32M, rk = e / kS32M;
        ps[e] = psih[(size_t)(w0 * KT + rk) * MP + m0 + m];
    }
    for (int e = tid; e < nw; e += kSpecThreads) lat[e] = wins[w0 + e].lat;
    // window-sum role: channel cs of the chunk, frequency ms
    const int cs = tid / kS32M, ms = tid % kS32M;
    // product role: channels cl + 32 r, frequencies 4 q .. 4 q + 3
    const int cl = tid / 8, q = tid % 8;
    float2 acc[COR][4];
#pragma unroll
    for (int r = 0; r < COR; ++r)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[r][u] = make_float2(0.0f, 0.0f);
#pragma unroll 1
    for (int c0 = 0; c0 < Ci; c0 += kS32C) {
        __syncthreads();   // the previous chunk's tile and weights are used (and ps, lat are in)
        for (int e = tid; e < Co * kS32C * KT; e += kSpecThreads) {
            const int co = e / (kS32C * KT), r = e - co * (kS32C * KT);
            const int ci = c0 + r / KT, k = r % KT;
            // wtr: w stored [Ci][Co][K] (the layer's weights, read by its adjoint)
            wt[e] = ci < Ci ? w[(wtr ? (size_t)ci * Co + co : (size_t)co * Ci + ci) * KT + k]
                            : 0.0f;
        }
        {
            const int ci = c0 + cs;
            float2 xa[KT];
#pragma unroll
            for (int k = 0; k < KT; ++k) xa[k] = make_float2(0.0f, 0.0f);
            if (ci < Ci) {
                const float2* xrow = xh + ((size_t)b * Ci + ci) * nlat_in * MP + m0 + ms;
                // four windows' samples loaded together, then used
#pragma unroll 1
                for (int w4 = 0; w4 < nw; w4 += 4) {
                    float2 xv[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        xv[u] = xrow[(size_t)lat[min(w4 + u, nw - 1)] * MP];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        if (w4 + u >= nw) break;
                        const int wi = w4 + u;
#pragma unroll
                        for (int k = 0; k < KT; ++k) {
                            const float2 P = ps[(wi * KT + k) * kS32M + ms];
                            // x_hat * conj(Psi_hat)
                            xa[k].x = fmaf(xv[u].x, P.x, fmaf(xv[u].y, P.y, xa[k].x));
                            xa[k].y = fmaf(xv[u].y, P.x, fmaf(-xv[u].x, P.y, xa[k].y));
                        }
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < KT; ++k) xt[(cs * KT + k) * kS32M + ms] = xa[k];
        }
        __syncthreads();
#pragma unroll 2
        for (int c = 0; c < kS32C; ++c) {
#pragma unroll
            for (int k = 0; k < KT; ++k) {
                const float4* xp = reinterpret_cast<const float4*>(xt + (c * KT + k) * kS32M + 4 * q);
                const float4 x01 = xp[0], x23 = xp[1];
                const float2 X[4] = {make_float2(x01.x, x01.y), make_float2(x01.z, x01.w),
                                     make_float2(x23.x, x23.y), make_float2(x23.z, x23.w)};
#pragma unroll
                for (int r = 0; r < COR; ++r) {
                    const int co = cl + 32 * r;
                    const float wv = co < Co ? wt[(co * kS32C + c) * KT + k] : 0.0f;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        acc[r][u].x = fmaf(wv, X[u].x, acc[r][u].x);
                        acc[r][u].y = fmaf(wv, X[u].y, acc[r][u].y);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < COR; ++r) {
        const int co = cl + 32 * r;
        if (co < Co) {
            float4* dst = reinterpret_cast<float4*>(
                yh + (((size_t)b * Co + co) * nlat_out + j) * MP + m0 + 4 * q);
            dst[0] = make_float4(acc[r][0].x, acc[r][0].y, acc[r][1].x, acc[r][1].y);
            dst[1] = make_float4(acc[r][2].x, acc[r][2].y, acc[r][3].x, acc[r][3].y);
        }
    }
}

// LDS bytes of spec32_conv
size_t spec32_lds(int K, int Co, int nwmax) {
    return ((size_t)nwmax * K * kS32M + (size_t)kS32C * K * kS32M) * sizeof(float2) +
           (size_t)Co * kS32C * K * sizeof(float) + (size_t)nwmax * sizeof(int);
}

}  // namespace

// Which fused algorithm disco_fused_fwd takes for these arguments.
int fused_spectral_eligible(const disco_psi* psi, int x_dtype, int Ci, int Co, int groups) {
    const DevPsi& d = psi->dev;
    const HostPsi& h = psi->host;
    if (x_dtype == DISCO_F32) {
        // float32, stride 1, up to 128 output channels, LDS of the vector kernel
        if (d.spec_mp <= 0 || d.spec_psih32 == nullptr || h.stride != 1 || groups != 1 ||
            h.K > 8 || Co > 128 || Ci < 1 || spec32_lds(h.K, Co, d.max_windows) > 64 * 1024)
            return 0;
        const char* e32 = std::getenv("DISCO_FUSED_PATH");
        return e32 == nullptr || std::strcmp(e32, "toeplitz") != 0;
    }
    if (d.spec_mp <= 0 || x_dtype != DISCO_BF16 || groups != 1 || Ci % 32 != 0 ||
        (Co != 128 && Co != 64) || h.K > 8)
        return 0;
    // the matrix-core kernel reads each row's first window, so every output
    // row needs one (a cap narrower than the input row spacing can miss
    // every input row)
    if (d.max_windows > kSpecMaxWin || d.min_windows < 1) return 0;
    // stride 2: register transforms on both sides (the tables exist only then)
    if (h.stride == 2 && h.desc.nlon_in != 1440 && h.desc.nlon_in != 720) return 0;
    // DISCO_FUSED_PATH=toeplitz selects the direct matrix-core kernel instead
    const char* e = std::getenv("DISCO_FUSED_PATH");
    return e == nullptr || std::strcmp(e, "toeplitz") != 0;
}

namespace {

// One bf16 longitude-spectral pass: rows of x (B x Ci planes of nin rows of
// N samples) -> x_hat; per output row (B x Co planes of nout rows) the window
// sums over its window list (win_ptr / wins, Psi_hat table psih in the list's
// order, multiplied conjugated) and the channel/basis GEMM; the inverse
// transform into y (+ bias).  The forward layer is (x, w, its windows,
// Psi_hat); its adjoint in x is (gy, w read transposed, the transposed
// windows, conj(Psi_hat) in their order), at stride 1.
struct SpecCall {
    const void* x;
    int nin;
    const void* w;
    int wt;                    // w stored [Ci][Co][K] (read transposed)
    const int32_t* win_ptr;
    const DevWindow* wins;
    size_t nwin;
    int max_windows, min_windows;
    const uint32_t* psih;
    const float* psih32;       // float32 layers: Psi_hat pairs in the list's order
    int nout;
    const float* bias;
    void* y;
    int y_dtype;
    int B, Ci, Co;
    int fold;       // longitude stride of the output (1, or 2: folded inverse)
    int upsample;   // x rows hold nlon_in / 2 samples: zero-inserted to nlon_in first
};

int run_spectral_bf16(const disco_psi* psi, const SpecCall& c, hipStream_t st, int* rc);

}  // namespace

int try_launch_fused_spectral(const disco_psi* psi, const void* x, const void* w,
                              const float* bias, void* y, int y_dtype, int B, int Ci, int Co,
                              int groups, hipStream_t st, int* rc) {
    if (!fused_spectral_eligible(psi, DISCO_BF16, Ci, Co, groups) || B <= 0) return 0;
    const DevPsi& d = psi->dev;
    const HostPsi& h = psi->host;
    SpecCall c{};
    c.x = x;
    c.nin = h.desc.nlat_in;
    c.w = w;
    c.wt = 0;
    c.win_ptr = d.win_ptr;
    c.wins = d.windows;
    c.nwin = h.windows.size();
    c.max_windows = d.max_windows;
    c.min_windows = d.min_windows;
    c.psih = static_cast<const uint32_t*>(d.spec_psih);
    c.nout = h.desc.nlat_out;
    c.bias = bias;
    c.y = y;
    c.y_dtype = y_dtype;
    c.B = B;
    c.Ci = Ci;
    c.Co = Co;
    c.fold = h.stride;
    c.upsample = 0;
    return run_spectral_bf16(psi, c, st, rc);
}

// The adjoint in x of the fused forward, for bf16 layers with bf16 gradients
// at stride 1 or 2 (the layers with spectral tables): gx = irfft(sum over
// output rows j and k of Psi_hat[k, j, i, m] sum_co w[co, ci, k]
// gy_hat[co, j, m]), on the forward's kernels; at stride 2 gy_hat is the
// spectrum of gy with zeros inserted between its samples.
int spectral_grad_x_eligible(const disco_psi* psi, int x_dtype, int gy_dtype, int Ci, int Co,
                             int groups) {
    const DevPsi& d = psi->dev;
    const HostPsi& h = psi->host;
    if (d.spec_psih_t == nullptr || (h.stride != 1 && h.stride != 2) || x_dtype != DISCO_BF16 ||
        gy_dtype != DISCO_BF16 || groups != 1 || h.K > 8 || Co % 32 != 0 ||
        (Ci != 64 && Ci != 128) || d.t_max_windows > kSpecMaxWin || d.t_min_windows < 1)
        return 0;
    const char* e = std::getenv("DISCO_FUSED_PATH");
    return e == nullptr || std::strcmp(e, "toeplitz") != 0;
}

int try_launch_grad_x_spectral(const disco_psi* psi, const void* gy, const void* w, void* gx,
                               int gx_dtype, int B, int Ci, int Co, hipStream_t st, int* rc) {
    if (!spectral_grad_x_eligible(psi, DISCO_BF16, DISCO_BF16, Ci, Co, 1) || B <= 0) return 0;
    const DevPsi& d = psi->dev;
    const HostPsi& h = psi->host;
    SpecCall c{};
    c.x = gy;
    c.nin = h.desc.nlat_out;
    c.w = w;
    c.wt = 1;
    c.win_ptr = d.wint_ptr;
    c.wins = d.wins_t;
    c.nwin = h.windows.size();
    c.max_windows = d.t_max_windows;
    c.min_windows = d.t_min_windows;
    c.psih = static_cast<const uint32_t*>(d.spec_psih_t);
    c.nout = h.desc.nlat_in;
    c.bias = nullptr;
    c.y = gx;
    c.y_dtype = gx_dtype;
    c.B = B;
    c.Ci = Co;   // the adjoint's GEMM maps the layer's output channels
    c.Co = Ci;   // to its input channels
    // stride 2: the adjoint of keeping every second longitude inserts zeros
    // between gy's samples, after which it is the stride-1 adjoint
    c.fold = 1;
    c.upsample = h.stride == 2;
    return run_spectral_bf16(psi, c, st, rc);
}

namespace {

int run_spectral_bf16(const disco_psi* psi, const SpecCall& c, hipStream_t st, int* rc) {
    const DevPsi& d = psi->dev;
    const HostPsi& h = psi->host;
    const disco_psi_desc& D = h.desc;
    const void* x = c.x;   // replaced by the zero-inserted rows (upsample)
    const void* w = c.w;
    const int wt = c.wt;
    const float* bias = c.bias;
    void* y = c.y;
    const int y_dtype = c.y_dtype, B = c.B, Ci = c.Ci, Co = c.Co;
    const int nlat_in = c.nin, nlat_out = c.nout;
    const int N = D.nlon_in, H = N / 2, MP = d.spec_mp, K = h.K;
    SpecPlan pl;
    pl.n = d.spec_nrad;
    for (int i = 0; i < kSpecMaxRadix; ++i) pl.r[i] = d.spec_radix[i];

    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t xh_bytes = up((size_t)B * Ci * nlat_in * MP * 4);
    const size_t yh_bytes = up((size_t)B * Co * nlat_out * MP * 4);
    const size_t wp_bytes = up((size_t)Co * Ci * 8 * 2);
    // zero-inserted rows (upsample): B Ci nlat_in rows of N bf16
    const size_t xu_bytes = c.upsample ? up((size_t)B * Ci * nlat_in * N * 2) : 0;
    const size_t ws_bytes = xh_bytes + yh_bytes + wp_bytes + xu_bytes;
    // the handle's workspace; stream-ordered memory while a graph is captured
    WorkspaceLease lease(psi, ws_bytes, st);
    if (lease.error() != DISCO_OK) {
        *rc = lease.error();
        return 1;
    }
    void* ws = lease.ptr();
    const bool own_ws = ws == nullptr;
    if (own_ws) {
        hipError_t e = hipMallocAsync(&ws, ws_bytes, st);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            *rc = set_error(e == hipErrorOutOfMemory ? DISCO_ENOMEM : DISCO_EHIP,
                            "hipMallocAsync for the spectral workspace failed: %s",
                            hipGetErrorString(e));
            return 1;
        }
    }
    uint32_t* xh = static_cast<uint32_t*>(ws);
    bf16_t* yh = reinterpret_cast<bf16_t*>(static_cast<char*>(ws) + xh_bytes);
    bf16_t* wpd = reinterpret_cast<bf16_t*>(static_cast<char*>(ws) + xh_bytes + yh_bytes);
    const uint32_t* psih = c.psih;
    if (c.upsample) {
        // word n of an upsampled row is the bf16 pair (gy[n], 0)
        uint32_t* xu = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + xh_bytes + yh_bytes +
                                                   wp_bytes);
        const size_t nw = (size_t)B * Ci * nlat_in * (N / 2);
        KernelTimer timer("spec_zero_insert", st);
        hipLaunchKernelGGL(spec_zero_insert, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, st,
                           static_cast<const bf16_t*>(x), xu, nw);
        x = xu;
    }

    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    (void)hipGetLastError();
    // the register-resident transforms cover these half lengths (their MP is
    // the table's)
    const bool reg = (H == 720 || H == 360 || H == 180) && MP == spec_mp_of(H);
    const int S = c.fold;   // 1, or 2 with register transforms on both sides (eligibility)
    // one-wave workgroups, one group of rw rows each
    auto reg_grid = [](int64_t rows, int rw) { return dim3((unsigned)((rows + rw - 1) / rw)); };

    const size_t nwp = (size_t)Co * Ci * 8;
    if (!reg) {
        KernelTimer timer("spec_prep_w", st);
        hipLaunchKernelGGL(spec_prep_w, dim3((unsigned)((nwp + 255) / 256)), dim3(256), 0, st,
                           static_cast<const bf16_t*>(w), wpd, Co, Ci, K, wt);
    }
    const size_t fft_lds = (size_t)(kFftRows + 1) * H * sizeof(float2);
    const int64_t xrows = (int64_t)B * Ci * nlat_in;
    const uint32_t* x32 = static_cast<const uint32_t*>(x);
    // the register transforms' launch also writes the weight fragments
    const int nprep = (int)((nwp + kPrepPerWg - 1) / kPrepPerWg);
#define DISCO_RF(H1, H2, RW)                                                                   \
    hipLaunchKernelGGL((spec_rfft_reg<H1, H2, RW>),                                            \
                       dim3((unsigned)(nprep + (xrows + RW - 1) / RW)),                        \
                       dim3(kRegThreads), 0, st, x32, xh, xrows,                               \
                       static_cast<const bf16_t*>(w), wpd, Co, Ci, K, nprep, wt)
    {
    KernelTimer timer("spec_rfft", st);
    if (reg && H == 720) {
        DISCO_RF(16, 45, 4);
    } else if (reg && H == 360) {
        DISCO_RF(8, 45, 8);
    } else if (reg && H == 180) {
        DISCO_RF(4, 45, 16);
    } else {
        hipLaunchKernelGGL((spec_rfft<bf16_t, uint32_t>),
                           dim3((unsigned)((xrows + kFftRows - 1) / kFftRows)), dim3(kFftThreads),
                           fft_lds, st, static_cast<const bf16_t*>(x), xh, N, MP, xrows, pl);
    }
    }
#undef DISCO_RF
    // bands of output rows, one per XCD; GX workgroups per band, at most the
    // smallest band's item count
    const int64_t nrows_all = (int64_t)B * nlat_out;
    const int NX = (int)std::min<int64_t>(kXcds, nrows_all);
    const int64_t min_items = nrows_all / NX * (MP / kMt);
    // window capacity: 8 (two workgroups per compute unit) or 16 (one).
    // Rows with 9 to 16 windows run on the 8-window kernel in two halves
    // (each item visited once per half of its windows, both accumulated
    // before y_hat is stored) when every row has at least two windows.
    const char* eh = std::getenv("DISCO_SPEC_HALVES");
    const bool halves = c.max_windows > 8 && c.min_windows >= 2 && !(eh && eh[0] == '0');
    const int NWC = c.max_windows <= 8 || halves ? 8 : 16;
    const int NPART = halves ? 2 : 1;
    const int nwmax = halves ? (c.max_windows + 1) / 2 : c.max_windows;
    const int per_cu = NWC == 8 ? 2 : 1;
    const int GX =
        (int)std::max<int64_t>(1, std::min<int64_t>(min_items, per_cu * (int64_t)ncu / NX));
    dim3 grid((unsigned)(NX * GX));
#define DISCO_SM(CC, KK, NWT)                                                                \
    hipLaunchKernelGGL((spec_mfma<CC, KK, NWT>), grid, dim3(kSpecThreads), 0, st, xh, wpd,   \
                       psih, c.win_ptr, c.wins, yh, B, Ci, nlat_in, nlat_out, MP, NX,           \
                       (int64_t)c.nwin * K * MP, nwmax, NPART)
#define DISCO_SM_K(CC, NWT)                                                                  \
    switch (K) {                                                                             \
        case 1: DISCO_SM(CC, 1, NWT); break;                                                 \
        case 2: DISCO_SM(CC, 2, NWT); break;                                                 \
        case 3: DISCO_SM(CC, 3, NWT); break;                                                 \
        case 4: DISCO_SM(CC, 4, NWT); break;                                                 \
        case 5: DISCO_SM(CC, 5, NWT); break;                                                 \
        case 6: DISCO_SM(CC, 6, NWT); break;                                                 \
        case 7: DISCO_SM(CC, 7, NWT); break;                                                 \
        default: DISCO_SM(CC, 8, NWT); break;                                                \
    }
    {
        KernelTimer timer("spec_mfma", st);
        if (Co == 128) {
            if (NWC == 8) {
                DISCO_SM_K(128, 8)
            } else {
                DISCO_SM_K(128, 16)
            }
        } else {
            if (NWC == 8) {
                DISCO_SM_K(64, 8)
            } else {
                DISCO_SM_K(64, 16)
            }
        }
    }
#undef DISCO_SM_K
#undef DISCO_SM
    const int64_t yrows = (int64_t)B * Co * nlat_out;
    const dim3 igrid((unsigned)((yrows + kFftRows - 1) / kFftRows));
    const uint32_t* yh32 = reinterpret_cast<const uint32_t*>(yh);
#define DISCO_IR(H1, H2, RW, TY, FD)                                                           \
    hipLaunchKernelGGL((spec_irfft_reg<H1, H2, RW, TY, FD>),                                   \
                       reg_grid(yrows, RW),                                                    \
                       dim3(kRegThreads), 0, st, yh32, static_cast<TY*>(y), bias, Co,          \
                       nlat_out, yrows, MP)
#define DISCO_IR_T(H1, H2, RW, FD)             \
    if (y_dtype == DISCO_F32) {                \
        DISCO_IR(H1, H2, RW, float, FD);       \
    } else {                                   \
        DISCO_IR(H1, H2, RW, bf16_t, FD);      \
    }
    {
    KernelTimer timer("spec_irfft", st);
    if (S == 2 && H == 720) {
        DISCO_IR_T(8, 45, 8, 2)          // 360-point half transform of the 720 outputs
    } else if (S == 2) {
        DISCO_IR_T(4, 45, 16, 2)         // H == 360: 180-point half transform
    } else if (reg && H == 720) {
        DISCO_IR_T(16, 45, 4, 1)
    } else if (reg && H == 360) {
        DISCO_IR_T(8, 45, 8, 1)
    } else if (reg && H == 180) {
        DISCO_IR_T(4, 45, 16, 1)
    } else if (y_dtype == DISCO_F32)
        hipLaunchKernelGGL((spec_irfft<uint32_t, float>), igrid, dim3(kFftThreads), fft_lds, st,
                           reinterpret_cast<const uint32_t*>(yh), static_cast<float*>(y), bias, N,
                           MP, Co, nlat_out, yrows, pl);
    else
        hipLaunchKernelGGL((spec_irfft<uint32_t, bf16_t>), igrid, dim3(kFftThreads), fft_lds, st,
                           reinterpret_cast<const uint32_t*>(yh), static_cast<bf16_t*>(y), bias, N,
                           MP, Co, nlat_out, yrows, pl);
    }
#undef DISCO_IR_T
#undef DISCO_IR
    hipError_t le = hipGetLastError();
    hipError_t fe = own_ws ? hipFreeAsync(ws, st) : hipSuccess;
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

}  // namespace

}  // namespace disco

namespace disco {

// The float32 spectral forward (stride 1): spec_rfft (float32 spectra),
// spec32_conv, spec_irfft.  Returns 0 when the layer does not qualify.
namespace {
int run_spectral_f32(const disco_psi* psi, const SpecCall& c, hipStream_t st, int* rc);
}  // namespace

int try_launch_fused_spectral32(const disco_psi* psi, const void* x, const void* w,
                                const float* bias, void* y, int y_dtype, int B, int Ci, int Co,
                                int groups, hipStream_t st, int* rc) {
    if (!fused_spectral_eligible(psi, DISCO_F32, Ci, Co, groups) || B <= 0) return 0;
    // rows are read and written as float pairs
    if ((reinterpret_cast<uintptr_t>(x) & 7) != 0 || (reinterpret_cast<uintptr_t>(y) & 7) != 0)
        return 0;
    const DevPsi& d = psi->dev;
    const HostPsi& h = psi->host;
    SpecCall c{};
    c.x = x;
    c.nin = h.desc.nlat_in;
    c.w = w;
    c.wt = 0;
    c.win_ptr = d.win_ptr;
    c.wins = d.windows;
    c.nwin = h.windows.size();
    c.max_windows = d.max_windows;
    c.min_windows = d.min_windows;
    c.psih32 = d.spec_psih32;
    c.nout = h.desc.nlat_out;
    c.bias = bias;
    c.y = y;
    c.y_dtype = y_dtype;
    c.B = B;
    c.Ci = Ci;
    c.Co = Co;
    c.fold = 1;
    return run_spectral_f32(psi, c, st, rc);
}

// The adjoint in x of the float32 spectral forward (stride 1, float32 x, w
// and gy): the transposed windows, conj(Psi_hat) in their order, the
// weights read transposed; float32 throughout.
int spectral_grad_x32_eligible(const disco_psi* psi, int Ci, int Co, int groups) {
    const DevPsi& d = psi->dev;
    const HostPsi& h = psi->host;
    if (d.spec_psih32_t == nullptr || h.stride != 1 || groups != 1 || h.K > 8 || Ci > 128 ||
        Co < 1 || d.t_min_windows < 1 || spec32_lds(h.K, Ci, d.t_max_windows) > 64 * 1024)
        return 0;
    const char* e = std::getenv("DISCO_FUSED_PATH");
    return e == nullptr || std::strcmp(e, "toeplitz") != 0;
}

int try_launch_grad_x_spectral32(const disco_psi* psi, const void* gy, const void* w, void* gx,
                                 int gx_dtype, int B, int Ci, int Co, hipStream_t st, int* rc) {
    if (!spectral_grad_x32_eligible(psi, Ci, Co, 1) || B <= 0) return 0;
    if ((reinterpret_cast<uintptr_t>(gy) & 7) != 0 || (reinterpret_cast<uintptr_t>(gx) & 7) != 0)
        return 0;
    const DevPsi& d = psi->dev;
    const HostPsi& h = psi->host;
    SpecCall c{};
    c.x = gy;
    c.nin = h.desc.nlat_out;
    c.w = w;
    c.wt = 1;
    c.win_ptr = d.wint_ptr;
    c.wins = d.wins_t;
    c.nwin = h.windows.size();
    c.max_windows = d.t_max_windows;
    c.min_windows = d.t_min_windows;
    c.psih32 = d.spec_psih32_t;
    c.nout = h.desc.nlat_in;
    c.bias = nullptr;
    c.y = gx;
    c.y_dtype = gx_dtype;
    c.B = B;
    c.Ci = Co;   // the adjoint maps the layer's output channels to its inputs
    c.Co = Ci;
    c.fold = 1;
    return run_spectral_f32(psi, c, st, rc);
}

namespace {

int run_spectral_f32(const disco_psi* psi, const SpecCall& c, hipStream_t st, int* rc) {
    const DevPsi& d = psi->dev;
    const HostPsi& h = psi->host;
    const disco_psi_desc& D = h.desc;
    const void* x = c.x;
    const void* w = c.w;
    const float* bias = c.bias;
    void* y = c.y;
    const int y_dtype = c.y_dtype, B = c.B, Ci = c.Ci, Co = c.Co;
    const int nlat_in = c.nin, nlat_out = c.nout;
    const int N = D.nlon_in, H = N / 2, MP = d.spec_mp, K = h.K;
    SpecPlan pl;
    pl.n = d.spec_nrad;
    for (int i = 0; i < kSpecMaxRadix; ++i) pl.r[i] = d.spec_radix[i];
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t xh_bytes = up((size_t)B * Ci * nlat_in * MP * sizeof(float2));
    const size_t yh_bytes = up((size_t)B * Co * nlat_out * MP * sizeof(float2));
    // the handle's workspace; stream-ordered memory while a graph is captured
    WorkspaceLease lease(psi, xh_bytes + yh_bytes, st);
    if (lease.error() != DISCO_OK) {
        *rc = lease.error();
        return 1;
    }
    void* ws = lease.ptr();
    const bool own_ws = ws == nullptr;
    if (own_ws) {
        hipError_t e = hipMallocAsync(&ws, xh_bytes + yh_bytes, st);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            *rc = set_error(e == hipErrorOutOfMemory ? DISCO_ENOMEM : DISCO_EHIP,
                            "hipMallocAsync for the spectral workspace failed: %s",
                            hipGetErrorString(e));
            return 1;
        }
    }
    float2* xh = static_cast<float2*>(ws);
    float2* yh = reinterpret_cast<float2*>(static_cast<char*>(ws) + xh_bytes);
    const size_t fft_lds = (size_t)(kFftRows + 1) * H * sizeof(float2);
    const int64_t xrows = (int64_t)B * Ci * nlat_in;
    {
        KernelTimer timer("spec_rfft", st);
        hipLaunchKernelGGL((spec_rfft<float, float2>),
                           dim3((unsigned)((xrows + kFftRows - 1) / kFftRows)), dim3(kFftThreads),
                           fft_lds, st, static_cast<const float*>(x), xh, N, MP, xrows, pl);
    }
    const int COR = (Co + 31) / 32;   // 1 .. 4 (Co <= 128)
    const size_t lds = spec32_lds(K, Co, c.max_windows);
    const dim3 grid((unsigned)((int64_t)B * nlat_out * (MP / kS32M)));
#define DISCO_S32(KK, CR)                                                                        \
    hipLaunchKernelGGL((spec32_conv<KK, CR>), grid, dim3(kSpecThreads), lds, st, xh,            \
                       static_cast<const float*>(w), reinterpret_cast<const float2*>(c.psih32), \
                       c.win_ptr, c.wins, yh, Ci, Co, nlat_in, nlat_out, MP, c.max_windows,     \
                       c.wt)
#define DISCO_S32_C(KK)                   \
    switch (COR) {                        \
        case 1: DISCO_S32(KK, 1); break;  \
        case 2: DISCO_S32(KK, 2); break;  \
        case 3: DISCO_S32(KK, 3); break;  \
        default: DISCO_S32(KK, 4); break; \
    }
    {
        KernelTimer timer("spec32_conv", st);
        switch (K) {
            case 1: DISCO_S32_C(1) break;
            case 2: DISCO_S32_C(2) break;
            case 3: DISCO_S32_C(3) break;
            case 4: DISCO_S32_C(4) break;
            case 5: DISCO_S32_C(5) break;
            case 6: DISCO_S32_C(6) break;
            case 7: DISCO_S32_C(7) break;
            default: DISCO_S32_C(8) break;
        }
    }
#undef DISCO_S32_C
#undef DISCO_S32
    const int64_t yrows = (int64_t)B * Co * nlat_out;
    const dim3 igrid((unsigned)((yrows + kFftRows - 1) / kFftRows));
    {
        KernelTimer timer("spec_irfft", st);
        if (y_dtype == DISCO_F32)
            hipLaunchKernelGGL((spec_irfft<float2, float>), igrid, dim3(kFftThreads), fft_lds, st,
                               yh, static_cast<float*>(y), bias, N, MP, Co, nlat_out, yrows, pl);
        else
            hipLaunchKernelGGL((spec_irfft<float2, bf16_t>), igrid, dim3(kFftThreads), fft_lds, st,
                               yh, static_cast<bf16_t*>(y), bias, N, MP, Co, nlat_out, yrows, pl);
    }
    hipError_t le = hipGetLastError();
    hipError_t fe = own_ws ? hipFreeAsync(ws, st) : hipSuccess;
    if (le != hipSuccess) {
        *rc = set_error(DISCO_EHIP, "float32 spectral launch failed: %s", hipGetErrorString(le));
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

}  // namespace

}  // namespace disco
