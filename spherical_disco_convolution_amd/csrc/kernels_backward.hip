// Gradients of the forward DISCO convolution (gfx950, wave64, vector ALUs,
// float32 accumulation).
//
// The forward equation of the DiscreteContinuousConvS2 page is linear in x
// and in w, so its gradients are the adjoints of its two linear maps:
//  * grad_xk[b, G*Ci/G + ci', k, j, q] = sum_{co in G} w[co, ci', k] gy[b, co, j, q]
//    (adjoint of the channel/basis sum in X_K)          -> einsum_grad_xk
//  * grad_w[co, ci', k] = sum_{b, j, q} gy[b, co, j, q] X_K[b, G(co)*Ci/G + ci', k, j, q]
//    (adjoint of the channel/basis sum in w)            -> grad_w_partial + reduce
//  * grad_x[b, c, i, (q s + p) mod nlon_in] += sum_k Psi[k, j, (i, p)] grad_xk[b, c, k, j, q]
//    (adjoint of the sparse contraction)                -> contract_t_kernel
// The page's fused mode recomputes X_K in the backward pass instead of
// storing it; disco_fused_bwd does that in slabs of output rows, so the whole
// K-expanded tensor never exists at once.
//
// Every kernel takes a window of output rows [row0, row0 + nrows): the
// K-expanded tensors it reads or writes hold only those rows ([B, C, K,
// nrows, nlon_out]); gy is always the whole [B, Co, nlat_out, nlon_out].
#include <hip/hip_runtime.h>

#include <algorithm>

#include "disco_internal.h"
#include "kernels_common.h"

namespace disco {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Adjoint of the contraction, gathered per input row (no atomics): one
// workgroup per (input row i, channel c, batch b) sums over the windows
// (j, i) of its transposed window list with j in the slab.  With
// d = (n - p_lo - t) mod nlon_in, output q = d / s receives tap t from input
// longitude n exactly when s divides d; walking t in steps of s from the
// first such tap moves q down by one each step.  The window's K rows of
// grad_xk (K x nlon_out floats) and a chunk of TC taps are staged in LDS.
// ---------------------------------------------------------------------------
template <typename TG, typename TO, int KP, int QR>
__global__ __launch_bounds__(kThreads) void contract_t_kernel(
    const TG* __restrict__ gxk, TO* __restrict__ gx, const int32_t* __restrict__ wt_ptr,
    const DevWindow* __restrict__ wt, const float* __restrict__ vals, int C, int K, int nlat_in,
    int nlon_in, int nlon_out, int s, int row0, int nrows, int accumulate, int TC) {
    extern __shared__ float smem[];
    float* G = smem;                              // [K][nlon_out]
    float* tp = smem + (size_t)K * nlon_out;      // [TC][KP]
    const int i = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
    const int w0 = wt_ptr[i], w1 = wt_ptr[i + 1];
    TO* out = gx + (((size_t)b * C + c) * nlat_in + i) * nlon_in;
    // windows of this input row whose output row lies in the slab (uniform)
    bool any = false;
    for (int wi = w0; wi < w1; ++wi) {
        const int jr = wt[wi].lat - row0;
        any = any || (jr >= 0 && jr < nrows);
    }
    if (accumulate && !any) return;
    for (int n0 = 0; n0 < nlon_in; n0 += kThreads * QR) {
        float acc[QR];
#pragma unroll
        for (int r = 0; r < QR; ++r) acc[r] = 0.0f;
        for (int wi = w0; wi < w1; ++wi) {
            const DevWindow wd = wt[wi];    // wd.lat is the output row j
            const int jr = wd.lat - row0;
            if (jr < 0 || jr >= nrows) continue;
            const TG* gsrc = gxk + (((size_t)b * C + c) * K * nrows + jr) * nlon_out;
            __syncthreads();   // the previous window's rows and taps are used
            for (int u = threadIdx.x; u < K * nlon_out; u += kThreads) {
                const int k = u / nlon_out, q = u - k * nlon_out;
                G[u] = load_f(gsrc, (size_t)k * nrows * nlon_out + q);
            }
            for (int t0 = 0; t0 < wd.width; t0 += TC) {
                const int tw = min(TC, wd.width - t0);
                if (t0 > 0) __syncthreads();   // the previous chunk's taps are used
                const float* v = vals + ((size_t)wd.val_off + t0) * KP;
                for (int u = threadIdx.x; u < tw * KP; u += kThreads) tp[u] = v[u];
                __syncthreads();
#pragma unroll
                for (int r = 0; r < QR; ++r) {
                    const int n = n0 + threadIdx.x + kThreads * r;
                    if (n >= nlon_in) continue;
                    int d0 = (n - wd.p_lo - t0) % nlon_in;
                    if (d0 < 0) d0 += nlon_in;
                    const int ts = d0 % s;
                    int q = (d0 - ts) / s;
                    float a = 0.0f;
                    for (int t = ts; t < tw; t += s) {
                        const float* tv = tp + t * KP;
#pragma unroll
                        for (int k = 0; k < KP; ++k)
                            if (k < K) a = fmaf(tv[k], G[k * nlon_out + q], a);
                        if (--q < 0) q += nlon_out;
                    }
                    acc[r] += a;
                }
            }
        }
#pragma unroll
        for (int r = 0; r < QR; ++r) {
            const int n = n0 + threadIdx.x + kThreads * r;
            if (n >= nlon_in) continue;
            const float prev = accumulate ? load_f(out, n) : 0.0f;
            store_f(out, n, prev + acc[r]);
        }
    }
}

// ---------------------------------------------------------------------------
// Adjoint in x for one input channel per group (m = Co/groups output channels
// per group): the weights fold into the taps, as in the forward's depthwise
// kernel, so gy is contracted directly without grad_xk:
//   gx[b, g, i, n] = sum_{co in g} sum_{windows (j, i)} sum_t
//                    (sum_k w[co, 0, k] Psi[k, j, (i, p_lo + t)]) gy[b, co, j, q]
// with the (n, t) -> q rule of contract_t_kernel.  One workgroup per (input
// row i, group g, batch b); per window and output channel the gy row and the
// folded taps are staged in LDS, so the inner loop is one LDS read and one
// multiply-add per tap (K of each in the unfolded form).
// ---------------------------------------------------------------------------
template <typename TG, typename TW, typename TO, int QR>
__global__ __launch_bounds__(kThreads) void contract_t_folded_kernel(
    const TG* __restrict__ gy, const TW* __restrict__ w, TO* __restrict__ gx,
    const int32_t* __restrict__ wt_ptr, const DevWindow* __restrict__ wt,
    const float* __restrict__ vals, int Co, int groups, int K, int KP, int nlat_in, int nlon_in,
    int nlat_out, int nlon_out, int s) {
    extern __shared__ float smem[];
    float* G = smem;                  // [nlon_out]: the gy row
    float* wk = smem + nlon_out;      // [K]: the output channel's weights
    float* f = wk + K;                // [width]: the folded taps
    const int i = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int m = Co / groups;
    const int w0 = wt_ptr[i], w1 = wt_ptr[i + 1];
    TO* out = gx + (((size_t)b * groups + g) * nlat_in + i) * nlon_in;
    for (int n0 = 0; n0 < nlon_in; n0 += kThreads * QR) {
        float acc[QR];
#pragma unroll
        for (int r = 0; r < QR; ++r) acc[r] = 0.0f;
        for (int cm = 0; cm < m; ++cm) {
            const int co = g * m + cm;
            for (int wi = w0; wi < w1; ++wi) {
                const DevWindow wd = wt[wi];   // wd.lat is the output row j
                const TG* grow = gy + (((size_t)b * Co + co) * nlat_out + wd.lat) * nlon_out;
                __syncthreads();   // the previous window's row and taps are used
                for (int u = tid; u < nlon_out; u += kThreads) G[u] = load_f(grow, u);
                if (tid < K) wk[tid] = load_f(w, (size_t)co * K + tid);
                __syncthreads();
                const float* v = vals + (size_t)wd.val_off * KP;
                for (int t = tid; t < wd.width; t += kThreads) {
                    float a = 0.0f;
                    for (int k = 0; k < K; ++k) a = fmaf(wk[k], v[(size_t)t * KP + k], a);
                    f[t] = a;
                }
                __syncthreads();
#pragma unroll
                for (int r = 0; r < QR; ++r) {
                    const int n = n0 + tid + kThreads * r;
                    if (n >= nlon_in) continue;
                    int d0 = (n - wd.p_lo) % nlon_in;
                    if (d0 < 0) d0 += nlon_in;
                    const int ts = d0 % s;
                    int q = (d0 - ts) / s;
                    float a = 0.0f;
                    for (int t = ts; t < wd.width; t += s) {
                        a = fmaf(f[t], G[q], a);
                        if (--q < 0) q += nlon_out;
                    }
                    acc[r] += a;
                }
            }
        }
#pragma unroll
        for (int r = 0; r < QR; ++r) {
            const int n = n0 + tid + kThreads * r;
            if (n < nlon_in) store_f(out, n, acc[r]);
        }
    }
}

// The same adjoint with register tiles, for strides S = 1 and 2 with
// nlon_in = S nlon_out.  A thread item owns the 8 outputs
// n = S (A0 + r) + P, r < 8.  For a window starting at p_lo these outputs
// see the taps of one parity p as a one-dimensional convolution:
// gx[n_r] += sum_u f[S u + p] gy[(a0 + r - u) mod nlon_out], with p and a0
// the same for all 8.  The window's folded taps are staged in LDS split by
// parity (zeros past the window), and the gy row with an offset of
// nlon_out + 8 so that every index of the convolution is in range without
// a modulo.  Per chunk of 8 taps an item reads 8 taps (16-byte loads) and
// 15 gy values for 64 multiply-adds.
constexpr int kCtR = 8;   // outputs per item and taps per chunk

template <typename TG, typename TW, typename TO, int S, int IT>
__global__ __launch_bounds__(kThreads) void contract_t_folded_tiled(
    const TG* __restrict__ gy, const TW* __restrict__ w, TO* __restrict__ gx,
    const int32_t* __restrict__ wt_ptr, const DevWindow* __restrict__ wt,
    const float* __restrict__ vals, int Co, int groups, int K, int KP, int nlat_in, int nlon_in,
    int nlat_out, int nlon_out, int GXN, int UWP) {
    extern __shared__ __attribute__((aligned(16))) float tsm[];
    float* gxs = tsm;               // [GXN]: gy row, gxs[m] = gy[(m - nlon_out - 8) mod nlon_out]
    float* fs = gxs + GXN;          // [S][UWP]: folded taps by parity, zeros past the window
    float* wk = fs + S * UWP;       // [K]
    const int i = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int mch = Co / groups;
    const int NB = (nlon_out + kCtR - 1) / kCtR;   // 8-output blocks per residue
    const int off = nlon_out + kCtR;
    const int w0 = wt_ptr[i], w1 = wt_ptr[i + 1];
    float acc[IT][kCtR];
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
        for (int r = 0; r < kCtR; ++r) acc[it][r] = 0.0f;
    for (int cm = 0; cm < mch; ++cm) {
        const int co = g * mch + cm;
        for (int wi = w0; wi < w1; ++wi) {
            const DevWindow wd = wt[wi];   // wd.lat is the output row j
            const TG* grow = gy + (((size_t)b * Co + co) * nlat_out + wd.lat) * nlon_out;
            __syncthreads();   // the previous window's row and taps are used
            for (int m = tid; m < GXN; m += kThreads)
                gxs[m] = load_f(grow, (size_t)((unsigned)(m + 2 * nlon_out - off) %
                                               (unsigned)nlon_out));
            if (tid < K) wk[tid] = load_f(w, (size_t)co * K + tid);
            __syncthreads();
            const float* v = vals + (size_t)wd.val_off * KP;
            for (int e = tid; e < S * UWP; e += kThreads) {
                const int p = e / UWP, u = e - p * UWP;
                const int t = S * u + p;
                float a = 0.0f;
                if (t < wd.width)
                    for (int k = 0; k < K; ++k) a = fmaf(wk[k], v[(size_t)t * KP + k], a);
                fs[e] = a;
            }
            __syncthreads();
            const int c = wd.p_lo / S, e0 = wd.p_lo - c * S;
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int item = tid + it * kThreads;
                if (item >= S * NB) continue;
                const int P = item / NB, A0 = (item - P * NB) * kCtR;
                const int p = P >= e0 ? P - e0 : P - e0 + S;
                int a0 = A0 - c - (P >= e0 ? 0 : 1);
                a0 %= nlon_out;
                if (a0 < 0) a0 += nlon_out;
                // taps of parity p in the window: u < up
                const int up = wd.width > p ? (wd.width - p + S - 1) / S : 0;
                const float* fp = fs + p * UWP;
                for (int u0 = 0; u0 < up; u0 += kCtR) {
                    float fv[kCtR];
#pragma unroll
                    for (int q = 0; q < kCtR / 4; ++q) {
                        const float4 x4 = *reinterpret_cast<const float4*>(fp + u0 + 4 * q);
                        fv[4 * q] = x4.x;
                        fv[4 * q + 1] = x4.y;
                        fv[4 * q + 2] = x4.z;
                        fv[4 * q + 3] = x4.w;
                    }
                    // gv[k] = gy[(a0 - u0 - 7 + k) mod nlon_out], k < 15
                    const float* gb = gxs + (a0 + off - u0 - (kCtR - 1));
                    float gv[2 * kCtR - 1];
#pragma unroll
                    for (int k = 0; k < 2 * kCtR - 1; ++k) gv[k] = gb[k];
#pragma unroll
                    for (int uu = 0; uu < kCtR; ++uu)
#pragma unroll
                        for (int r = 0; r < kCtR; ++r)
                            acc[it][r] = fmaf(fv[uu], gv[r - uu + kCtR - 1], acc[it][r]);
                }
            }
        }
    }
    TO* out = gx + (((size_t)b * groups + g) * nlat_in + i) * nlon_in;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int item = tid + it * kThreads;
        if (item >= S * NB) continue;
        const int P = item / NB, A0 = (item - P * NB) * kCtR;
#pragma unroll
        for (int r = 0; r < kCtR; ++r)
            if (A0 + r < nlon_out) store_f(out, (size_t)S * (A0 + r) + P, acc[it][r]);
    }
}

// ---------------------------------------------------------------------------
// grad_w partial sums on the matrix cores, for a bf16 gy and one group: a
// 128 x 128 tile of [co][kappa] over one chunk of points; four waves of
// 64 x 64, each 2 x 2 v_mfma_f32_32x32x16_bf16 per 16 points.  The operands
// load straight from memory along the point axis (lane l: row l % 32 of its
// tile, points 8 (l / 32) .. + 7 of the step: 16 bytes of gy, 32 bytes of a
// float32 X_K rounded to bf16 as it is loaded).  partial[(b nchunk +
// chunk)][co][kappa], the layout of grad_w_partial.
// ---------------------------------------------------------------------------
typedef __bf16 gw_bf16x8 __attribute__((ext_vector_type(8)));
typedef float gw_floatx16 __attribute__((ext_vector_type(16)));
constexpr int kGwM = 128;   // tile edge of the matrix-core kernel

__device__ __forceinline__ gw_bf16x8 gw_load8(const bf16_t* p) {
    return *reinterpret_cast<const gw_bf16x8*>(p);
}
__device__ __forceinline__ gw_bf16x8 gw_load8(const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    typedef float f8 __attribute__((ext_vector_type(8)));
    const f8 v = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    return __builtin_convertvector(v, gw_bf16x8);   // round to nearest even
}

template <typename TX>
__global__ __launch_bounds__(kThreads) void grad_w_mfma(
    const TX* __restrict__ xk, const bf16_t* __restrict__ gy, float* __restrict__ partial, int Co,
    int kd, int nlat_out, int nlon_out, int row0, int nrows, int L, int nchunk) {
    const int kt = blockIdx.x, ct = blockIdx.y;
    const int z = blockIdx.z;
    const int chunk = z % nchunk, b = z / nchunk;
    const size_t P = (size_t)nrows * nlon_out;   // points of the slab
    const size_t n0 = (size_t)chunk * L;
    const size_t n1 = min(P, n0 + (size_t)L);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, lg = lane >> 5;
    const int co0 = ct * kGwM + (wave & 1) * 64, ka0 = kt * kGwM + (wave >> 1) * 64;
    const bf16_t* gyb = gy + (size_t)b * Co * nlat_out * nlon_out + (size_t)row0 * nlon_out;
    const TX* xkb = xk + (size_t)b * kd * P;
    const bf16_t* arow[2];
    const TX* brow[2];
    bool aok[2], bok[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int co = co0 + 32 * u + l32, ka = ka0 + 32 * u + l32;
        aok[u] = co < Co;
        bok[u] = ka < kd;
        arow[u] = gyb + (size_t)min(co, Co - 1) * nlat_out * nlon_out;
        brow[u] = xkb + (size_t)min(ka, kd - 1) * P;
    }
    gw_floatx16 acc[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[u][v][e] = 0.0f;
    const gw_bf16x8 zero = {};
    for (size_t nb = n0; nb < n1; nb += 16) {
        // P, L and the chunk starts are multiples of 8: a lane's 8 points
        // are all inside the chunk or all past it
        const size_t p = nb + 8 * lg;
        const bool pin = p + 8 <= n1;
        gw_bf16x8 af[2], bf[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            af[u] = aok[u] && pin ? gw_load8(arow[u] + p) : zero;
            bf[u] = bok[u] && pin ? gw_load8(brow[u] + p) : zero;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int v = 0; v < 2; ++v)
                acc[u][v] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[u], bf[v], acc[u][v], 0, 0, 0);
    }
    // lane: column kappa = ka0 + 32 v + l32, rows co = co0 + 32 u + 8 (e / 4) + 4 lg + e % 4
    float* out = partial + (size_t)(b * nchunk + chunk) * Co * kd;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const int ka = ka0 + 32 * v + l32;
            if (ka >= kd) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int co = co0 + 32 * u + 8 * (e >> 2) + 4 * lg + (e & 3);
                if (co < Co) out[(size_t)co * kd + ka] = acc[u][v][e];
            }
        }
}

// The same partial sums from a bf16 X_K, staged through LDS: per step of 64
// points the workgroup copies 128 bytes of each of its tile's 128 gy rows and
// 128 X_K rows into LDS (8 lanes per row, 16 bytes per lane: whole row
// segments, each row read once for the four waves), then every wave runs its
// 2 x 2 MFMAs over the step's four 16-point slices from there.  The next
// step's rows are loaded into registers while the MFMAs run.
constexpr int kGwP = 64;            // points per staged step
constexpr int kGwPitch = kGwP + 8;  // LDS row pitch in bf16 (144 bytes)

__global__ __launch_bounds__(kThreads) void grad_w_mfma_lds(
    const bf16_t* __restrict__ xk, const bf16_t* __restrict__ gy, float* __restrict__ partial,
    int Co, int kd, int nlat_out, int nlon_out, int row0, int nrows, int L, int nchunk) {
    __shared__ __attribute__((aligned(16))) bf16_t sa[kGwM * kGwPitch];   // gy rows of the tile
    __shared__ __attribute__((aligned(16))) bf16_t sb[kGwM * kGwPitch];   // X_K rows of the tile
    const int kt = blockIdx.x, ct = blockIdx.y;
    const int z = blockIdx.z;
    const int chunk = z % nchunk, b = z / nchunk;
    const size_t P = (size_t)nrows * nlon_out;   // points of the slab
    const size_t n0 = (size_t)chunk * L;
    const size_t n1 = min(P, n0 + (size_t)L);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, lg = lane >> 5;
    // staging: thread tid copies 8-point piece tid % 8 of tile rows tid / 8 + 32 r
    const int piece = tid & 7, srow = tid >> 3;
    const bf16_t* gyb = gy + (size_t)b * Co * nlat_out * nlon_out + (size_t)row0 * nlon_out;
    const bf16_t* xkb = xk + (size_t)b * kd * P;
    const bf16_t* asrc[4];
    const bf16_t* bsrc[4];
    bool aok[4], bok[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int co = ct * kGwM + srow + 32 * r, ka = kt * kGwM + srow + 32 * r;
        aok[r] = co < Co;
        bok[r] = ka < kd;
        asrc[r] = gyb + (size_t)min(co, Co - 1) * nlat_out * nlon_out;
        bsrc[r] = xkb + (size_t)min(ka, kd - 1) * P;
    }
    const gw_bf16x8 zero = {};
    gw_bf16x8 ra[4], rb[4];
    // P, L and the chunk starts are multiples of 8: a piece's 8 points are
    // all inside the chunk or all past it (then zeros, which add nothing)
    auto fetch = [&](size_t nb) {
        const size_t p = nb + 8 * piece;
        const bool pin = p + 8 <= n1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            ra[r] = aok[r] && pin ? gw_load8(asrc[r] + p) : zero;
            rb[r] = bok[r] && pin ? gw_load8(bsrc[r] + p) : zero;
        }
    };
    const int am = (wave & 1) * 64, bm = (wave >> 1) * 64;   // the wave's 64 x 64 sub-tile
    gw_floatx16 acc[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[u][v][e] = 0.0f;
    if (n0 < n1) fetch(n0);
    for (size_t nb = n0; nb < n1; nb += kGwP) {
        __syncthreads();   // every wave is done reading the previous step
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            *reinterpret_cast<gw_bf16x8*>(sa + (srow + 32 * r) * kGwPitch + 8 * piece) = ra[r];
            *reinterpret_cast<gw_bf16x8*>(sb + (srow + 32 * r) * kGwPitch + 8 * piece) = rb[r];
        }
        __syncthreads();
        if (nb + kGwP < n1) fetch(nb + kGwP);   // in flight during this step's MFMAs
#pragma unroll
        for (int s = 0; s < kGwP / 16; ++s) {
            gw_bf16x8 af[2], bf[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                af[u] = *reinterpret_cast<const gw_bf16x8*>(sa + (am + 32 * u + l32) * kGwPitch +
                                                            16 * s + 8 * lg);
                bf[u] = *reinterpret_cast<const gw_bf16x8*>(sb + (bm + 32 * u + l32) * kGwPitch +
                                                            16 * s + 8 * lg);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int v = 0; v < 2; ++v)
                    acc[u][v] =
                        __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[u], bf[v], acc[u][v], 0, 0, 0);
        }
    }
    // lane: column kappa = ka0 + 32 v + l32, rows co = co0 + 32 u + 8 (e / 4) + 4 lg + e % 4
    const int co0 = ct * kGwM + am, ka0 = kt * kGwM + bm;
    float* out = partial + (size_t)(b * nchunk + chunk) * Co * kd;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const int ka = ka0 + 32 * v + l32;
            if (ka >= kd) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int co = co0 + 32 * u + 8 * (e >> 2) + 4 * lg + (e & 3);
                if (co < Co) out[(size_t)co * kd + ka] = acc[u][v][e];
            }
        }
}

// ---------------------------------------------------------------------------
// grad_w of layers with one input channel per group, with no X_K.  For output
// channel co (input channel c = co / (Co / groups)) and basis function k,
//   gw[co, 0, k] = sum_{b, j} sum_{windows (i, p_lo) of row j} sum_t
//                  Psi_k[window, t] * S[t],
//   S[t] = sum_q gy[b, co, j, q] * x[b, c, i, (s q + p_lo + t) mod nlon_in].
// One workgroup per (output row, output channel, batch).  Per window the
// input row's samples from p_lo on are staged in LDS by residue mod s
// (ext_p[m] = sample p_lo + s m + p), so output t = s a + p at tap q reads
// ext_p[a + q].  Thread items are (8 consecutive a, a slice of q) with an
// 8 x 8 register tile per residue; each item's S values go to LDS per q
// slice; then one thread per t sums the slices and folds S[t] with the
// window's K values into its gw registers.  A workgroup reduction writes
// partial[(b nlat_out + j)][co][k], which reduce_partials sums in order.
// ---------------------------------------------------------------------------
constexpr int kDwgR = 8;        // register tile edge
constexpr int kDwgMaxK = 32;    // largest K
constexpr int kDwgSlices = 16;  // most q slices per window

template <typename TX, typename TG, int S>
__global__ __launch_bounds__(kThreads) void grad_w_depthwise(
    const TX* __restrict__ x, const TG* __restrict__ gy, float* __restrict__ partial,
    const int32_t* __restrict__ win_ptr, const DevWindow* __restrict__ wins,
    const float* __restrict__ vals, int Co, int groups, int K, int KP, int nlat_in, int nlon_in,
    int nlat_out, int nlon_out, int QP, int GQ, int M4, int area) {
    extern __shared__ __attribute__((aligned(16))) float dsm[];
    float* gys = dsm;             // [GQ >= QP]: gy row j, zeros past nlon_out
    float* ext = gys + GQ;        // [S][M4]
    float* sl = ext + S * M4;     // [area]: S values per q slice
    const int j = blockIdx.x, co = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int c = co / (Co / groups);
    const TG* gyr = gy + (((size_t)b * Co + co) * nlat_out + j) * nlon_out;
    const TX* xc = x + ((size_t)b * groups + c) * nlat_in * nlon_in;
    for (int q = tid; q < QP; q += kThreads) gys[q] = q < nlon_out ? load_f(gyr, q) : 0.0f;
    float gwk[kDwgMaxK];
#pragma unroll
    for (int k = 0; k < kDwgMaxK; ++k) gwk[k] = 0.0f;
    const int nqb = QP / kDwgR;   // q blocks
    const int w0 = win_ptr[j], w1 = win_ptr[j + 1];
    for (int wi = w0; wi < w1; ++wi) {
        const DevWindow wd = wins[wi];
        if (wd.width <= 0) continue;     // uniform over the workgroup
        const int A = (wd.width + S - 1) / S;
        const int NA = (A + kDwgR - 1) / kDwgR;
        const int M = NA * kDwgR + QP;   // ext_p entries the items read
        const int TW = S * NA * kDwgR;   // t entries per slice
        // at most kDwgSlices slices: the fold below sums them serially per t
        const int NQ = max(1, min(min(min(nqb, kThreads / NA), area / TW), kDwgSlices));
        const int qbs = (nqb + NQ - 1) / NQ;   // q blocks per slice
        const TX* row = xc + (size_t)wd.lat * nlon_in;
        __syncthreads();   // the previous window's reads are done; gys is written
        // sample p_lo + u (mod nlon_in): reduced once, then advanced by
        // kThreads per step (a while loop: rows may be shorter than kThreads)
        int pos = (int)(((unsigned)wd.p_lo + (unsigned)tid) % (unsigned)nlon_in);
        for (int u = tid; u < S * M; u += kThreads) {
            const int m = u / S, p = u - m * S;
            ext[p * M4 + m] = load_f(row, pos);
            pos += kThreads;
            while (pos >= nlon_in) pos -= nlon_in;
        }
        __syncthreads();
        for (int it = tid; it < NA * NQ; it += kThreads) {
            const int ab = it % NA, qs = it / NA;
            const int a0 = ab * kDwgR;
            const int qa = qs * qbs * kDwgR, qb = min(QP, qa + qbs * kDwgR);
            float acc[S][kDwgR];
#pragma unroll
            for (int p = 0; p < S; ++p)
#pragma unroll
                for (int r = 0; r < kDwgR; ++r) acc[p][r] = 0.0f;
            for (int q = qa; q < qb; q += kDwgR) {
                float g[kDwgR];
#pragma unroll
                for (int i = 0; i < kDwgR / 4; ++i) {
                    const float4 v = *reinterpret_cast<const float4*>(gys + q + 4 * i);
                    g[4 * i] = v.x;
                    g[4 * i + 1] = v.y;
                    g[4 * i + 2] = v.z;
                    g[4 * i + 3] = v.w;
                }
#pragma unroll
                for (int p = 0; p < S; ++p) {
                    // ext_p[a0 + q .. a0 + q + 15]: a0 + q is a multiple of 8
                    float e[2 * kDwgR];
#pragma unroll
                    for (int i = 0; i < 2 * kDwgR / 4; ++i) {
                        const float4 v =
                            *reinterpret_cast<const float4*>(ext + p * M4 + a0 + q + 4 * i);
                        e[4 * i] = v.x;
                        e[4 * i + 1] = v.y;
                        e[4 * i + 2] = v.z;
                        e[4 * i + 3] = v.w;
                    }
#pragma unroll
                    for (int u = 0; u < kDwgR; ++u)
#pragma unroll
                        for (int r = 0; r < kDwgR; ++r) acc[p][r] = fmaf(g[u], e[r + u], acc[p][r]);
                }
            }
            float* dst = sl + qs * TW;
#pragma unroll
            for (int p = 0; p < S; ++p)
#pragma unroll
                for (int r = 0; r < kDwgR; ++r) dst[S * (a0 + r) + p] = acc[p][r];
        }
        __syncthreads();
        const float* v = vals + (size_t)wd.val_off * KP;
        for (int t = tid; t < wd.width; t += kThreads) {
            float st = 0.0f;
            for (int qs = 0; qs < NQ; ++qs) st += sl[qs * TW + t];
#pragma unroll
            for (int k = 0; k < kDwgMaxK; ++k)
                if (k < K) gwk[k] = fmaf(v[(size_t)t * KP + k], st, gwk[k]);
        }
    }
    // workgroup sum of gwk: lane shuffles within each wave, then LDS
    __syncthreads();
    float* red = dsm;   // [kThreads / 64][kDwgMaxK], inside gys (GQ >= 4 kDwgMaxK)
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int k = 0; k < kDwgMaxK; ++k) {
        if (k < K) {
            float a = gwk[k];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) a += __shfl_xor(a, off);
            if (lane == 0) red[wave * kDwgMaxK + k] = a;
        }
    }
    __syncthreads();
    if (tid < K) {
        float a = 0.0f;
        for (int w = 0; w < kThreads / 64; ++w) a += red[w * kDwgMaxK + tid];
        partial[((size_t)(b * nlat_out + j) * Co + co) * K + tid] = a;
    }
}

// ---------------------------------------------------------------------------
// grad_w partial sums: a 64 x 64 tile of [co in group][kappa = (ci', k)]
// summed over one chunk of L output points (r, q) of one batch entry,
// staged 16 points at a time through LDS; thread = 4 x 4 outputs.
// partial[(b * nchunk + chunk)][co][kappa], co over all groups.
// ---------------------------------------------------------------------------
constexpr int kGwT = 64;   // tile edge
constexpr int kGwS = 16;   // points per step
template <typename TX, typename TG>
__global__ __launch_bounds__(kThreads) void grad_w_partial(
    const TX* __restrict__ xk, const TG* __restrict__ gy, float* __restrict__ partial, int Ci,
    int Co, int groups, int K, int nlat_out, int nlon_out, int row0, int nrows, int L,
    int nchunk) {
    __shared__ float As[kGwS][kGwT + 4];   // gy[co][n]
    __shared__ float Bs[kGwS][kGwT + 4];   // xk[kappa][n]
    const int cig = Ci / groups, cog = Co / groups;
    const int kd = cig * K;
    const int kt = blockIdx.x, ct = blockIdx.y;
    const int z = blockIdx.z;
    const int chunk = z % nchunk;
    const int bg = z / nchunk;
    const int g = bg % groups, b = bg / groups;
    const size_t P = (size_t)nrows * nlon_out;   // points of the slab
    const size_t n0 = (size_t)chunk * L;
    const size_t n1 = min(P, n0 + (size_t)L);
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    // load roles: element e = threadIdx.x + 256 u (u < 4) of the 64 x 16 tile:
    // row e / 16, point e % 16
    const TG* gyb = gy + ((size_t)b * Co + (size_t)g * cog) * nlat_out * nlon_out +
                    (size_t)row0 * nlon_out;
    const TX* xkb = xk + ((size_t)b * Ci + (size_t)g * cig) * K * P;
    float acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[a][e] = 0.0f;
    for (size_t nb = n0; nb < n1; nb += kGwS) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = threadIdx.x + kThreads * u;
            const int row = e / kGwS, p = e % kGwS;
            const size_t n = nb + p;
            const int co = ct * kGwT + row;
            const int kap = kt * kGwT + row;
            As[p][row] = (co < cog && n < n1)
                             ? load_f(gyb, (size_t)co * nlat_out * nlon_out + n)
                             : 0.0f;
            Bs[p][row] = (kap < kd && n < n1) ? load_f(xkb, (size_t)kap * P + n) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < kGwS; ++p) {
            float av[4], bv[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) av[a] = As[p][ty + 16 * a];
#pragma unroll
            for (int e = 0; e < 4; ++e) bv[e] = Bs[p][tx + 16 * e];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[a][e] = fmaf(av[a], bv[e], acc[a][e]);
        }
        __syncthreads();
    }
    float* out = partial + (size_t)(b * nchunk + chunk) * Co * kd;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int co = ct * kGwT + ty + 16 * a;
        if (co >= cog) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int kap = kt * kGwT + tx + 16 * e;
            if (kap < kd) out[((size_t)g * cog + co) * kd + kap] = acc[a][e];
        }
    }
}

// gw[e] (+)= sum over the nparts partial arrays of e, in a fixed order
__global__ __launch_bounds__(kThreads) void reduce_partials(const float* __restrict__ partial,
                                                            float* __restrict__ gw, size_t n,
                                                            int nparts, int accumulate) {
    const size_t e = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (e >= n) return;
    float a = accumulate ? gw[e] : 0.0f;
    for (int p = 0; p < nparts; ++p) a += partial[(size_t)p * n + e];
    gw[e] = a;
}

// ---------------------------------------------------------------------------
// grad_xk for a slab: thread = output point n of the slab plane, COT pairs
// (ci', k) of one group per workgroup row; weights are wave-uniform.
//   gxk[b, g cig + ci', k, r, q] = sum_{co' < cog} w[g cog + co', ci', k] gy[b, g cog + co', row0 + r, q]
// ---------------------------------------------------------------------------
template <typename TG, typename TW, typename TO, int COT>
__global__ __launch_bounds__(kThreads) void einsum_grad_xk_kernel(
    const TG* __restrict__ gy, const TW* __restrict__ w, TO* __restrict__ gxk, int Ci, int Co,
    int groups, int K, int nlat_out, int nlon_out, int row0, int nrows) {
    const int cig = Ci / groups, cog = Co / groups;
    const int kd = cig * K;
    const size_t P = (size_t)nrows * nlon_out;
    const size_t n = (size_t)blockIdx.x * kThreads + threadIdx.x;
    const int oc0 = blockIdx.y * COT;      // first (ci, k) pair over all groups: ci * K + k
    const int b = blockIdx.z;
    const int g = oc0 / kd;
    if (n >= P) return;
    float acc[COT];
#pragma unroll
    for (int c = 0; c < COT; ++c) acc[c] = 0.0f;
    const TG* gyb = gy + ((size_t)b * Co + (size_t)g * cog) * nlat_out * nlon_out +
                    (size_t)row0 * nlon_out + n;
    const int kap0 = oc0 - g * kd;          // (ci', k) within the group
    for (int co = 0; co < cog; ++co) {
        const float gv = load_f(gyb, (size_t)co * nlat_out * nlon_out);
        const TW* wr = w + ((size_t)g * cog + co) * kd + kap0;
#pragma unroll
        for (int c = 0; c < COT; ++c) acc[c] = fmaf(load_f(wr, c), gv, acc[c]);
    }
    // gxk layout [B, Ci, K, nrows, nlon_out]: pair oc = ci * K + k is plane oc
    TO* out = gxk + ((size_t)b * Ci * K + oc0) * P + n;
#pragma unroll
    for (int c = 0; c < COT; ++c) store_f(out, (size_t)c * P, acc[c]);
}

// grad_bias[co] = sum_{b, j, q} gy[b, co, j, q]: one workgroup per co, fixed
// order (per-thread strided sums, then a tree over the workgroup)
template <typename TG>
__global__ __launch_bounds__(kThreads) void grad_bias_kernel(const TG* __restrict__ gy,
                                                             float* __restrict__ gb, int B, int Co,
                                                             size_t HW) {
    __shared__ float red[kThreads];
    const int co = blockIdx.x;
    float a = 0.0f;
    for (int b = 0; b < B; ++b) {
        const TG* p = gy + ((size_t)b * Co + co) * HW;
        for (size_t n = threadIdx.x; n < HW; n += kThreads) a += load_f(p, n);
    }
    red[threadIdx.x] = a;
    __syncthreads();
    for (int h = kThreads / 2; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) gb[co] = red[0];
}

// float32 zeros (graph-capturable: no memset node)
__global__ __launch_bounds__(kThreads) void fill_zero(float* __restrict__ p, size_t n) {
    const size_t e = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (e < n) p[e] = 0.0f;
}

int check(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return set_error(DISCO_EHIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return DISCO_OK;
}

int pick_qr_t(int nlon_in) {
    const int qr = (nlon_in + kThreads - 1) / kThreads;
    return qr <= 1 ? 1 : qr <= 2 ? 2 : qr <= 3 ? 3 : qr <= 4 ? 4 : qr <= 6 ? 6 : 8;
}

// LDS of the transposed contraction: K rows of grad_xk plus TC taps; the
// largest TC (256 down to 16) that keeps it within 64 KiB, or 0.
int pick_tc(int K, int KP, int nlon_out, size_t* lds) {
    for (int tc = 256; tc >= 16; tc /= 2) {
        const size_t bytes = ((size_t)K * nlon_out + (size_t)tc * KP) * sizeof(float);
        if (bytes <= 64 * 1024) {
            *lds = bytes;
            return tc;
        }
    }
    return 0;
}

template <typename TG, typename TO, int KP>
int contract_t_kp(const disco_psi* psi, const void* gxk, void* gx, int B, int C, int row0,
                  int nrows, int accumulate, hipStream_t st) {
    const HostPsi& h = psi->host;
    const DevPsi& d = psi->dev;
    const disco_psi_desc& D = h.desc;
    size_t lds = 0;
    const int TC = pick_tc(h.K, KP, D.nlon_out, &lds);
    if (TC == 0)
        return set_error(DISCO_EUNSUPPORTED, "K * nlon_out = %d too large for the transposed "
                         "contraction (K rows of one output row must fit in 64 KiB)",
                         h.K * D.nlon_out);
    const int QR = pick_qr_t(D.nlon_in);
    dim3 grid(D.nlat_in, C, B);
#define DISCO_CT(Q)                                                                              \
    hipLaunchKernelGGL((contract_t_kernel<TG, TO, KP, Q>), grid, dim3(kThreads), lds, st,        \
                       (const TG*)gxk, (TO*)gx, d.wint_ptr, d.wins_t, d.vals, C, h.K, D.nlat_in,  \
                       D.nlon_in, D.nlon_out, h.stride, row0, nrows, accumulate, TC)
    KernelTimer timer("contract_transpose", st);
    switch (QR) {
        case 1: DISCO_CT(1); break;
        case 2: DISCO_CT(2); break;
        case 3: DISCO_CT(3); break;
        case 4: DISCO_CT(4); break;
        case 6: DISCO_CT(6); break;
        default: DISCO_CT(8); break;
    }
#undef DISCO_CT
    return check("contract_transpose");
}

template <typename TG, typename TO>
int contract_t_dispatch(const disco_psi* psi, const void* gxk, void* gx, int B, int C, int row0,
                        int nrows, int accumulate, hipStream_t st) {
    switch (psi->dev.KP) {
#define DISCO_CTK(N) \
    case N: return contract_t_kp<TG, TO, N>(psi, gxk, gx, B, C, row0, nrows, accumulate, st);
        DISCO_CTK(1) DISCO_CTK(2) DISCO_CTK(4) DISCO_CTK(8) DISCO_CTK(12) DISCO_CTK(16)
        DISCO_CTK(20) DISCO_CTK(24) DISCO_CTK(28) DISCO_CTK(32)
#undef DISCO_CTK
        default:
            return set_error(DISCO_EUNSUPPORTED, "K = %d is not supported by the transposed "
                             "contraction (K <= 32)", psi->host.K);
    }
}

int contract_t_any(const disco_psi* psi, const void* gxk, int gxk_dtype, void* gx, int gx_dtype,
                   int B, int C, int row0, int nrows, int accumulate, hipStream_t st) {
    if (gxk_dtype == DISCO_F32 && gx_dtype == DISCO_F32)
        return contract_t_dispatch<float, float>(psi, gxk, gx, B, C, row0, nrows, accumulate, st);
    if (gxk_dtype == DISCO_F32)
        return contract_t_dispatch<float, bf16_t>(psi, gxk, gx, B, C, row0, nrows, accumulate, st);
    if (gx_dtype == DISCO_F32)
        return contract_t_dispatch<bf16_t, float>(psi, gxk, gx, B, C, row0, nrows, accumulate, st);
    return contract_t_dispatch<bf16_t, bf16_t>(psi, gxk, gx, B, C, row0, nrows, accumulate, st);
}

// points per grad_w chunk: enough workgroups to fill the chip at least twice
// The matrix-core grad_w kernel takes bf16 gy (a bf16 gradient asks for the
// bf16 bar: X_K is rounded to bf16 as it is loaded), one group, and rows and
// chunks of whole 16-byte pieces.
bool grad_w_mfma_ok(int xk_dtype, int gy_dtype, int groups, int nlon_out, int L, const void* gy) {
    return gy_dtype == DISCO_BF16 && (xk_dtype == DISCO_F32 || xk_dtype == DISCO_BF16) &&
           groups == 1 && nlon_out % 8 == 0 && L % 16 == 0 &&
           (reinterpret_cast<uintptr_t>(gy) & 15) == 0;
}

// output tiles of one group's grad_w for the chunk split: 128 x 128 on the
// matrix cores, 64 x 64 otherwise
int grad_w_tiles(int gy_dtype, int groups, int cig, int cog, int K, int nlon_out) {
    if (gy_dtype == DISCO_BF16 && groups == 1 && nlon_out % 8 == 0)
        return ((cig * K + kGwM - 1) / kGwM) * ((cog + kGwM - 1) / kGwM);
    return ((cig * K + kGwT - 1) / kGwT) * ((cog + kGwT - 1) / kGwT);
}

int grad_w_chunk(size_t P, int tiles, int B, int groups, int ncu) {
    const size_t want = (size_t)2 * ncu;
    size_t per = (size_t)tiles * B * groups;
    size_t nchunk = std::max<size_t>(1, (want + per - 1) / per);
    size_t L = (P + nchunk - 1) / nchunk;
    L = std::max<size_t>(L, 1024);
    L = (L + kGwS - 1) / kGwS * kGwS;
    return (int)std::min<size_t>(L, (size_t)1 << 30);
}

int num_cus() {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    (void)hipGetLastError();
    return ncu;
}

// grad_w partial sums of one slab into `partial` ([B nchunk][Co][cig K]);
// returns the number of partial arrays written, or a negative error code
int grad_w_slab(const void* xk, int xk_dtype, const void* gy, int gy_dtype, float* partial,
                int B, int Ci, int Co, int groups, int K, int nlat_out, int nlon_out, int row0,
                int nrows, int L, hipStream_t st) {
    const int cig = Ci / groups, cog = Co / groups;
    const size_t P = (size_t)nrows * nlon_out;
    const int nchunk = (int)((P + L - 1) / L);
    if (grad_w_mfma_ok(xk_dtype, gy_dtype, groups, nlon_out, L, gy)) {
        const int kd = Ci * K;
        dim3 mgrid((kd + kGwM - 1) / kGwM, (Co + kGwM - 1) / kGwM, (unsigned)(B * nchunk));
        {
            KernelTimer timer("grad_w_mfma", st);
            if (xk_dtype == DISCO_F32)
                hipLaunchKernelGGL((grad_w_mfma<float>), mgrid, dim3(kThreads), 0, st,
                                   (const float*)xk, (const bf16_t*)gy, partial, Co, kd, nlat_out,
                                   nlon_out, row0, nrows, L, nchunk);
            else
                hipLaunchKernelGGL(grad_w_mfma_lds, mgrid, dim3(kThreads), 0, st,
                                   (const bf16_t*)xk, (const bf16_t*)gy, partial, Co, kd, nlat_out,
                                   nlon_out, row0, nrows, L, nchunk);
        }
        const int rc = check("grad_w_mfma");
        return rc != DISCO_OK ? rc : B * nchunk;
    }
    dim3 grid((cig * K + kGwT - 1) / kGwT, (cog + kGwT - 1) / kGwT, (unsigned)(B * groups * nchunk));
#define DISCO_GW(TX, TG)                                                                          \
    hipLaunchKernelGGL((grad_w_partial<TX, TG>), grid, dim3(kThreads), 0, st, (const TX*)xk,      \
                       (const TG*)gy, partial, Ci, Co, groups, K, nlat_out, nlon_out, row0, nrows, \
                       L, nchunk)
    {
        KernelTimer timer("grad_w_partial", st);
        if (xk_dtype == DISCO_F32 && gy_dtype == DISCO_F32) DISCO_GW(float, float);
        else if (xk_dtype == DISCO_F32) DISCO_GW(float, bf16_t);
        else if (gy_dtype == DISCO_F32) DISCO_GW(bf16_t, float);
        else DISCO_GW(bf16_t, bf16_t);
    }
#undef DISCO_GW
    int rc = check("grad_w_partial");
    return rc != DISCO_OK ? rc : B * nchunk;
}

int reduce_into(const float* partial, float* gw, size_t n, int nparts, int accumulate,
                hipStream_t st) {
    {
        KernelTimer timer("reduce_partials", st);
        hipLaunchKernelGGL(reduce_partials, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, st, partial, gw, n, nparts, accumulate);
    }
    return check("reduce_partials");
}

template <typename TG, typename TW, typename TO>
int grad_xk_typed(const void* gy, const void* w, void* gxk, int B, int Ci, int Co, int groups,
                  int K, int nlat_out, int nlon_out, int row0, int nrows, hipStream_t st) {
    const int kd = (Ci / groups) * K;
    int cot = 8;
    while (kd % cot) cot /= 2;
    const size_t P = (size_t)nrows * nlon_out;
    dim3 grid((unsigned)((P + kThreads - 1) / kThreads), (unsigned)(Ci * K / cot), (unsigned)B);
#define DISCO_GX(N)                                                                             \
    hipLaunchKernelGGL((einsum_grad_xk_kernel<TG, TW, TO, N>), grid, dim3(kThreads), 0, st,     \
                       (const TG*)gy, (const TW*)w, (TO*)gxk, Ci, Co, groups, K, nlat_out,      \
                       nlon_out, row0, nrows)
    KernelTimer timer("einsum_grad_xk", st);
    switch (cot) {
        case 8: DISCO_GX(8); break;
        case 4: DISCO_GX(4); break;
        case 2: DISCO_GX(2); break;
        default: DISCO_GX(1); break;
    }
#undef DISCO_GX
    return check("einsum_grad_xk");
}

int grad_xk_any(const void* gy, int gy_dtype, const void* w, int w_dtype, void* gxk, int gxk_dtype,
                int B, int Ci, int Co, int groups, int K, int nlat_out, int nlon_out, int row0,
                int nrows, hipStream_t st) {
#define DISCO_GXT(TG, TW, TO) \
    return grad_xk_typed<TG, TW, TO>(gy, w, gxk, B, Ci, Co, groups, K, nlat_out, nlon_out, row0, nrows, st)
    const bool g32 = gy_dtype == DISCO_F32, w32 = w_dtype == DISCO_F32, o32 = gxk_dtype == DISCO_F32;
    if (g32 && w32 && o32) DISCO_GXT(float, float, float);
    if (g32 && w32) DISCO_GXT(float, float, bf16_t);
    if (g32 && o32) DISCO_GXT(float, bf16_t, float);
    if (g32) DISCO_GXT(float, bf16_t, bf16_t);
    if (w32 && o32) DISCO_GXT(bf16_t, float, float);
    if (w32) DISCO_GXT(bf16_t, float, bf16_t);
    if (o32) DISCO_GXT(bf16_t, bf16_t, float);
    DISCO_GXT(bf16_t, bf16_t, bf16_t);
#undef DISCO_GXT
}

}  // namespace

int launch_fill_zero(float* p, size_t n, void* stream) {
    if (n == 0) return DISCO_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    {
        KernelTimer timer("fill_zero", st);
        hipLaunchKernelGGL(fill_zero, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads),
                           0, st, p, n);
    }
    return check("fill_zero");
}

// the contraction into an fp32 slab of output rows (kernels_generic.hip)

int launch_contract_rows(const disco_psi* psi, const void* x, int x_dtype, float* xk, int B, int C,
                         int row0, int nrows, hipStream_t st);

// The folded adjoint in x over the whole layer (one input channel per group).
template <typename TG, typename TW, typename TO>
int contract_t_folded_t(const disco_psi* psi, const void* gy, const void* w, void* gx, int B,
                        int Co, int groups, hipStream_t st) {
    const HostPsi& h = psi->host;
    const DevPsi& d = psi->dev;
    const disco_psi_desc& D = h.desc;
    const size_t lds = ((size_t)D.nlon_out + h.K + d.max_width) * sizeof(float);
    if (lds > 64 * 1024)
        return set_error(DISCO_EUNSUPPORTED, "rows too long for the folded transposed contraction");
    const int q0 = pick_qr_t(D.nlon_in);
    const int QR = q0 <= 1 ? 1 : q0 <= 2 ? 2 : q0 <= 4 ? 4 : 8;
    dim3 grid(D.nlat_in, groups, B);
#define DISCO_CTF(Q)                                                                          \
    hipLaunchKernelGGL((contract_t_folded_kernel<TG, TW, TO, Q>), grid, dim3(kThreads), lds, st, \
                       (const TG*)gy, (const TW*)w, (TO*)gx, d.wint_ptr, d.wins_t, d.vals, Co,  \
                       groups, h.K, d.KP, D.nlat_in, D.nlon_in, D.nlat_out, D.nlon_out, h.stride)
    KernelTimer timer("contract_transpose_folded", st);
    switch (QR) {
        case 1: DISCO_CTF(1); break;
        case 2: DISCO_CTF(2); break;
        case 4: DISCO_CTF(4); break;
        default: DISCO_CTF(8); break;
    }
#undef DISCO_CTF
    return check("contract_transpose_folded");
}

template <typename TG, typename TW>
int contract_t_folded_o(const disco_psi* psi, const void* gy, const void* w, void* gx,
                        int gx_dtype, int B, int Co, int groups, hipStream_t st) {
    return gx_dtype == DISCO_F32
               ? contract_t_folded_t<TG, TW, float>(psi, gy, w, gx, B, Co, groups, st)
               : contract_t_folded_t<TG, TW, bf16_t>(psi, gy, w, gx, B, Co, groups, st);
}

// The register-tiled form: returns 0 when the layer is not one it takes
// (stride 1 or 2 with nlon_in = S nlon_out, at most two items per thread, the
// LDS within 64 KiB), else 1 with *rc the result.
template <typename TG, typename TW, typename TO>
int contract_t_folded_tiled_t(const disco_psi* psi, const void* gy, const void* w, void* gx, int B,
                              int Co, int groups, hipStream_t st, int* rc) {
    const HostPsi& h = psi->host;
    const DevPsi& d = psi->dev;
    const disco_psi_desc& D = h.desc;
    const int S = h.stride;
    if ((S != 1 && S != 2) || D.nlon_in != S * D.nlon_out || d.max_width < 1 ||
        D.nlon_out < kCtR)
        return 0;
    const int NB = (D.nlon_out + kCtR - 1) / kCtR;
    const int IT = (S * NB + kThreads - 1) / kThreads;
    if (IT > 2) return 0;
    // gy indices a0 + off - u0 - 7 + k: a0 < nlon_out, u0 < UWP, k < 15
    const int UWP = ((d.max_width + S - 1) / S + kCtR - 1) / kCtR * kCtR;
    const int GXN = (2 * D.nlon_out + 2 * kCtR + 3) / 4 * 4;
    if (UWP > D.nlon_out + kCtR) return 0;
    const size_t lds = ((size_t)GXN + (size_t)S * UWP + h.K) * sizeof(float);
    if (lds > 64 * 1024) return 0;
    dim3 grid(D.nlat_in, groups, B);
#define DISCO_CTT(SS, II)                                                                       \
    hipLaunchKernelGGL((contract_t_folded_tiled<TG, TW, TO, SS, II>), grid, dim3(kThreads), lds, \
                       st, (const TG*)gy, (const TW*)w, (TO*)gx, d.wint_ptr, d.wins_t, d.vals,   \
                       Co, groups, h.K, d.KP, D.nlat_in, D.nlon_in, D.nlat_out, D.nlon_out, GXN, \
                       UWP)
    {
        KernelTimer timer("contract_transpose_folded_tiled", st);
        if (S == 1 && IT == 1) DISCO_CTT(1, 1);
        else if (S == 1) DISCO_CTT(1, 2);
        else if (IT == 1) DISCO_CTT(2, 1);
        else DISCO_CTT(2, 2);
    }
#undef DISCO_CTT
    *rc = check("contract_transpose_folded_tiled");
    return 1;
}

template <typename TG, typename TW>
int contract_t_folded_tiled_o(const disco_psi* psi, const void* gy, const void* w, void* gx,
                              int gx_dtype, int B, int Co, int groups, hipStream_t st, int* rc) {
    return gx_dtype == DISCO_F32
               ? contract_t_folded_tiled_t<TG, TW, float>(psi, gy, w, gx, B, Co, groups, st, rc)
               : contract_t_folded_tiled_t<TG, TW, bf16_t>(psi, gy, w, gx, B, Co, groups, st, rc);
}

int contract_t_folded(const disco_psi* psi, const void* gy, int gy_dtype, const void* w,
                      int w_dtype, void* gx, int gx_dtype, int B, int Co, int groups,
                      hipStream_t st) {
    int trc = DISCO_OK;
    int took;
    if (gy_dtype == DISCO_F32)
        took = w_dtype == DISCO_F32
                   ? contract_t_folded_tiled_o<float, float>(psi, gy, w, gx, gx_dtype, B, Co,
                                                             groups, st, &trc)
                   : contract_t_folded_tiled_o<float, bf16_t>(psi, gy, w, gx, gx_dtype, B, Co,
                                                              groups, st, &trc);
    else
        took = w_dtype == DISCO_F32
                   ? contract_t_folded_tiled_o<bf16_t, float>(psi, gy, w, gx, gx_dtype, B, Co,
                                                              groups, st, &trc)
                   : contract_t_folded_tiled_o<bf16_t, bf16_t>(psi, gy, w, gx, gx_dtype, B, Co,
                                                               groups, st, &trc);
    if (took) return trc;
    if (gy_dtype == DISCO_F32)
        return w_dtype == DISCO_F32
                   ? contract_t_folded_o<float, float>(psi, gy, w, gx, gx_dtype, B, Co, groups, st)
                   : contract_t_folded_o<float, bf16_t>(psi, gy, w, gx, gx_dtype, B, Co, groups, st);
    return w_dtype == DISCO_F32
               ? contract_t_folded_o<bf16_t, float>(psi, gy, w, gx, gx_dtype, B, Co, groups, st)
               : contract_t_folded_o<bf16_t, bf16_t>(psi, gy, w, gx, gx_dtype, B, Co, groups, st);
}

int launch_contract_transpose(const disco_psi* psi, const void* gxk, int gxk_dtype, void* gx,
                              int gx_dtype, int B, int C, void* stream) {
    return contract_t_any(psi, gxk, gxk_dtype, gx, gx_dtype, B, C, 0, psi->host.desc.nlat_out, 0,
                          static_cast<hipStream_t>(stream));
}

int launch_einsum_grad_xk(const void* gy, int gy_dtype, const void* w, int w_dtype, void* gxk,
                          int gxk_dtype, int B, int Ci, int Co, int groups, int K, int nlat_out,
                          int nlon_out, void* stream) {
    return grad_xk_any(gy, gy_dtype, w, w_dtype, gxk, gxk_dtype, B, Ci, Co, groups, K, nlat_out,
                       nlon_out, 0, nlat_out, static_cast<hipStream_t>(stream));
}

int launch_einsum_grad_w(const void* xk, int xk_dtype, const void* gy, int gy_dtype, float* gw,
                         int B, int Ci, int Co, int groups, int K, int nlat_out, int nlon_out,
                         void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int cig = Ci / groups, cog = Co / groups;
    const int tiles = grad_w_tiles(gy_dtype, groups, cig, cog, K, nlon_out);
    const size_t P = (size_t)nlat_out * nlon_out;
    const int L = grad_w_chunk(P, tiles, B, groups, num_cus());
    const int nparts = B * (int)((P + L - 1) / L);
    const size_t n = (size_t)Co * cig * K;
    void* ws = nullptr;
    hipError_t e = hipMallocAsync(&ws, (size_t)nparts * n * sizeof(float), st);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return set_error(e == hipErrorOutOfMemory ? DISCO_ENOMEM : DISCO_EHIP,
                         "hipMallocAsync for the grad_w partial sums failed: %s",
                         hipGetErrorString(e));
    }
    float* partial = static_cast<float*>(ws);
    int rc = grad_w_slab(xk, xk_dtype, gy, gy_dtype, partial, B, Ci, Co, groups, K, nlat_out,
                         nlon_out, 0, nlat_out, L, st);
    if (rc >= 0) rc = reduce_into(partial, gw, n, nparts, 0, st);
    hipError_t fe = hipFreeAsync(ws, st);
    if (rc != DISCO_OK) return rc;
    if (fe != hipSuccess) {
        (void)hipGetLastError();
        return set_error(DISCO_EHIP, "hipFreeAsync failed: %s", hipGetErrorString(fe));
    }
    return DISCO_OK;
}

// Fused-mode backward: per slab of output rows, X_K (float32) is recomputed
// from x, grad_w partial sums of the slab are reduced into gw, grad_xk of the
// slab is formed from gy and w, and its transposed contraction is added into
// gx.  Slabs of at most ceil(nlat_out / 8) rows (one slab when the two slab
// tensors of the whole layer take at most 64 MiB), so the workspace is about
// an eighth of the two whole K-expanded tensors.
// Largest bf16 X_K the fused backward recomputes whole on the matrix cores
// (1.86 GB for 128 channels, K = 7 at 721 x 1440); larger layers take the
// float32 slabs.
constexpr size_t kWholeXk16Max = (size_t)4 << 30;

// grad_w of a bf16 layer with a bf16 gradient and one group: the matrix-core
// contraction writes the whole bf16 X_K into the handle's workspace, the
// matrix-core partial sums run over every point, and one reduction writes gw.
// Returns 0 when the layer is not one this takes (rc untouched), else 1 with
// *rc the result.
// grad_w of a layer with one input channel per group (stride 1 or 2) with no
// X_K: grad_w_depthwise into per-(batch, output row) partials in the
// handle's workspace, then one reduction into gw.  Returns 0 when the layer
// is not one this takes (rc untouched), else 1 with *rc the result.
template <typename TX, typename TG>
void launch_grad_w_depthwise(const disco_psi* psi, const void* x, const void* gy, float* partial,
                             int B, int Co, int groups, int QP, int GQ, int M4, int area,
                             size_t lds, hipStream_t st) {
    const HostPsi& h = psi->host;
    const DevPsi& d = psi->dev;
    const disco_psi_desc& D = h.desc;
    dim3 grid(D.nlat_out, Co, B);
#define DISCO_GWD(SS)                                                                             \
    hipLaunchKernelGGL((grad_w_depthwise<TX, TG, SS>), grid, dim3(kThreads), lds, st,             \
                       (const TX*)x, (const TG*)gy, partial, d.win_ptr, d.windows, d.vals, Co,    \
                       groups, h.K, d.KP, D.nlat_in, D.nlon_in, D.nlat_out, D.nlon_out, QP, GQ,  \
                       M4, area)
    if (h.stride == 1) DISCO_GWD(1);
    else DISCO_GWD(2);
#undef DISCO_GWD
}

static int grad_w_depthwise_run(const disco_psi* psi, const void* x, int x_dtype, const void* gy,
                                int gy_dtype, float* gw, int B, int Co, int groups,
                                hipStream_t st, int* rc) {
    const HostPsi& h = psi->host;
    const DevPsi& d = psi->dev;
    const disco_psi_desc& D = h.desc;
    const int S = h.stride, K = h.K;
    if ((S != 1 && S != 2) || K > kDwgMaxK || B <= 0 || d.max_width < 1) return 0;
    const int QP = (D.nlon_out + kDwgR - 1) / kDwgR * kDwgR;
    const int GQ = std::max(QP, 4 * kDwgMaxK);
    const int NA = ((d.max_width + S - 1) / S + kDwgR - 1) / kDwgR;
    const int M4 = (NA * kDwgR + QP + 3) / 4 * 4;
    const int area = std::max(S * NA * kDwgR, 4096);
    const size_t lds = ((size_t)GQ + (size_t)S * M4 + area) * sizeof(float);
    if (lds > 64 * 1024) return 0;
    const int nparts = B * D.nlat_out;
    const size_t n = (size_t)Co * K;
    const size_t part_bytes = (size_t)nparts * n * sizeof(float);
    WorkspaceLease lease(psi, part_bytes, st);
    if (lease.error() != DISCO_OK) {
        *rc = lease.error();
        return 1;
    }
    void* ws = lease.ptr();
    const bool own_ws = ws == nullptr;
    if (own_ws) {
        hipError_t e = hipMallocAsync(&ws, part_bytes, st);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            *rc = set_error(e == hipErrorOutOfMemory ? DISCO_ENOMEM : DISCO_EHIP,
                            "hipMallocAsync for the backward workspace failed: %s",
                            hipGetErrorString(e));
            return 1;
        }
    }
    float* partial = static_cast<float*>(ws);
    {
        KernelTimer timer("grad_w_depthwise", st);
        if (x_dtype == DISCO_F32 && gy_dtype == DISCO_F32)
            launch_grad_w_depthwise<float, float>(psi, x, gy, partial, B, Co, groups, QP, GQ, M4,
                                                  area, lds, st);
        else if (x_dtype == DISCO_F32)
            launch_grad_w_depthwise<float, bf16_t>(psi, x, gy, partial, B, Co, groups, QP, GQ, M4,
                                                   area, lds, st);
        else if (gy_dtype == DISCO_F32)
            launch_grad_w_depthwise<bf16_t, float>(psi, x, gy, partial, B, Co, groups, QP, GQ, M4,
                                                   area, lds, st);
        else
            launch_grad_w_depthwise<bf16_t, bf16_t>(psi, x, gy, partial, B, Co, groups, QP, GQ,
                                                    M4, area, lds, st);
    }
    int r = check("grad_w_depthwise");
    if (r == DISCO_OK) r = reduce_into(partial, gw, n, nparts, 0, st);
    hipError_t fe = own_ws ? hipFreeAsync(ws, st) : hipSuccess;
    if (r == DISCO_OK && fe != hipSuccess) {
        (void)hipGetLastError();
        r = set_error(DISCO_EHIP, "hipFreeAsync failed: %s", hipGetErrorString(fe));
    }
    *rc = r;
    return 1;
}

static int grad_w_whole_bf16(const disco_psi* psi, const void* x, const void* gy, float* gw, int B,
                      int Ci, int Co, hipStream_t st, int* rc) {
    const HostPsi& h = psi->host;
    const disco_psi_desc& D = h.desc;
    const int K = h.K;
    const size_t P = (size_t)D.nlat_out * D.nlon_out;
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t xk_bytes = up((size_t)B * Ci * K * P * sizeof(bf16_t));
    if (xk_bytes > kWholeXk16Max) return 0;
    const int tiles = grad_w_tiles(DISCO_BF16, 1, Ci, Co, K, D.nlon_out);
    const int L = grad_w_chunk(P, tiles, B, 1, num_cus());
    // the workspace is 256-byte aligned: only x's alignment is in question
    if (!contract_mfma_ok(psi, x, x, B, Ci) || !grad_w_mfma_ok(DISCO_BF16, DISCO_BF16, 1,
                                                               D.nlon_out, L, gy))
        return 0;
    const int nparts = B * (int)((P + L - 1) / L);
    const size_t ngw = (size_t)Co * Ci * K;
    const size_t part_bytes = up((size_t)nparts * ngw * sizeof(float));
    WorkspaceLease lease(psi, xk_bytes + part_bytes, st);
    if (lease.error() != DISCO_OK) {
        *rc = lease.error();
        return 1;
    }
    void* ws = lease.ptr();
    const bool own_ws = ws == nullptr;
    if (own_ws) {
        hipError_t e = hipMallocAsync(&ws, xk_bytes + part_bytes, st);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            *rc = set_error(e == hipErrorOutOfMemory ? DISCO_ENOMEM : DISCO_EHIP,
                            "hipMallocAsync for the backward workspace failed: %s",
                            hipGetErrorString(e));
            return 1;
        }
    }
    bf16_t* xk = static_cast<bf16_t*>(ws);
    float* partial = reinterpret_cast<float*>(static_cast<char*>(ws) + xk_bytes);
    int r = DISCO_OK;
    if (!try_launch_contract_mfma(psi, x, xk, B, Ci, st, &r))
        r = set_error(DISCO_EHIP, "matrix-core contraction declined a layer it was checked for");
    if (r == DISCO_OK) {
        const int np = grad_w_slab(xk, DISCO_BF16, gy, DISCO_BF16, partial, B, Ci, Co, 1, K,
                                   D.nlat_out, D.nlon_out, 0, D.nlat_out, L, st);
        r = np < 0 ? np : reduce_into(partial, gw, ngw, np, 0, st);
    }
    hipError_t fe = own_ws ? hipFreeAsync(ws, st) : hipSuccess;
    if (r == DISCO_OK && fe != hipSuccess) {
        (void)hipGetLastError();
        r = set_error(DISCO_EHIP, "hipFreeAsync failed: %s", hipGetErrorString(fe));
    }
    *rc = r;
    return 1;
}

int launch_fused_bwd(const disco_psi* psi, const void* x, int x_dtype, const void* w, int w_dtype,
                     const void* gy, int gy_dtype, void* gx, int gx_dtype, float* gw, float* gbias,
                     int B, int Ci, int Co, int groups, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    const HostPsi& h = psi->host;
    const disco_psi_desc& D = h.desc;
    // bf16 layers with spectral tables and a bf16 gradient: grad_x on the
    // spectral kernels (the convolution adjoint of each window's
    // correlation), whole
    if (gx && x_dtype == DISCO_BF16 && w_dtype == DISCO_BF16 &&
        spectral_grad_x_eligible(psi, x_dtype, gy_dtype, Ci, Co, groups)) {
        int src = DISCO_OK;
        if (try_launch_grad_x_spectral(psi, gy, w, gx, gx_dtype, B, Ci, Co, st, &src)) {
            if (src != DISCO_OK) return src;
            gx = nullptr;
        }
    }
    // float32 stride-1 layers with a float32 gradient: the same on the float32
    // spectral kernels (float32 spectra: the float32 bar)
    if (gx && x_dtype == DISCO_F32 && w_dtype == DISCO_F32 && gy_dtype == DISCO_F32 &&
        spectral_grad_x32_eligible(psi, Ci, Co, groups)) {
        int src = DISCO_OK;
        if (try_launch_grad_x_spectral32(psi, gy, w, gx, gx_dtype, B, Ci, Co, st, &src)) {
            if (src != DISCO_OK) return src;
            gx = nullptr;
        }
    }
    const int K = h.K, cig = Ci / groups, cog = Co / groups;
    // one input channel per group: grad_x with the weights folded into the
    // taps, over the whole layer (no grad_xk)
    if (gx && cig == 1 && B > 0) {
        const int frc = contract_t_folded(psi, gy, gy_dtype, w, w_dtype, gx, gx_dtype, B, Co,
                                          groups, st);
        if (frc != DISCO_OK) return frc;
        gx = nullptr;
    }
    // bf16 x and gy, one group: X_K recomputed whole, in bf16, by the
    // matrix-core contraction, then the matrix-core grad_w partial sums over
    // every point (they hold X_K to bf16 as they load it in any case)
    if (gw && B > 0 && x_dtype == DISCO_BF16 && gy_dtype == DISCO_BF16 && groups == 1) {
        int grc = DISCO_OK;
        if (grad_w_whole_bf16(psi, x, gy, gw, B, Ci, Co, st, &grc)) {
            if (grc != DISCO_OK) return grc;
            gw = nullptr;
        }
    }
    // one input channel per group: grad_w straight from x and gy, no X_K
    if (gw && B > 0 && cig == 1) {
        int grc = DISCO_OK;
        if (grad_w_depthwise_run(psi, x, x_dtype, gy, gy_dtype, gw, B, Co, groups, st, &grc)) {
            if (grc != DISCO_OK) return grc;
            gw = nullptr;
        }
    }
    const size_t row_bytes = (size_t)B * Ci * K * D.nlon_out * sizeof(float);
    int rows = D.nlat_out;
    if ((size_t)2 * row_bytes * D.nlat_out > ((size_t)64 << 20)) rows = (D.nlat_out + 7) / 8;
    const int nslab = (D.nlat_out + rows - 1) / rows;
    const int tiles = grad_w_tiles(gy_dtype, groups, cig, cog, K, D.nlon_out);
    const int L = grad_w_chunk((size_t)rows * D.nlon_out, tiles, B, groups, num_cus());
    const int nparts_max = B * (int)(((size_t)rows * D.nlon_out + L - 1) / L);
    const size_t ngw = (size_t)Co * cig * K;
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t slab_bytes = up((size_t)rows * row_bytes);
    const size_t xk_bytes = gw ? slab_bytes : 0;
    const size_t gxk_bytes = gx ? slab_bytes : 0;
    const size_t part_bytes = gw ? up((size_t)nparts_max * ngw * sizeof(float)) : 0;
    void* ws = nullptr;
    int rc = DISCO_OK;
    if (gbias) {
        {
            KernelTimer timer("grad_bias", st);
            if (gy_dtype == DISCO_F32)
                hipLaunchKernelGGL(grad_bias_kernel<float>, dim3(Co), dim3(kThreads), 0, st,
                                   (const float*)gy, gbias, B, Co, (size_t)D.nlat_out * D.nlon_out);
            else
                hipLaunchKernelGGL(grad_bias_kernel<bf16_t>, dim3(Co), dim3(kThreads), 0, st,
                                   (const bf16_t*)gy, gbias, B, Co, (size_t)D.nlat_out * D.nlon_out);
        }
        if ((rc = check("grad_bias")) != DISCO_OK) return rc;
    }
    if (!gw && !gx) return DISCO_OK;
    // the handle's workspace; stream-ordered memory while a graph is captured
    WorkspaceLease lease(psi, xk_bytes + gxk_bytes + part_bytes, st);
    if (lease.error() != DISCO_OK) return lease.error();
    ws = lease.ptr();
    const bool own_ws = ws == nullptr;
    if (own_ws) {
        hipError_t e = hipMallocAsync(&ws, xk_bytes + gxk_bytes + part_bytes, st);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return set_error(e == hipErrorOutOfMemory ? DISCO_ENOMEM : DISCO_EHIP,
                             "hipMallocAsync for the backward workspace failed: %s",
                             hipGetErrorString(e));
        }
    }
    float* xk = static_cast<float*>(ws);
    float* gxk = reinterpret_cast<float*>(static_cast<char*>(ws) + xk_bytes);
    float* partial = reinterpret_cast<float*>(static_cast<char*>(ws) + xk_bytes + gxk_bytes);
    for (int sidx = 0; sidx < nslab && rc == DISCO_OK; ++sidx) {
        const int row0 = sidx * rows;
        const int nr = std::min(rows, D.nlat_out - row0);
        if (gw) {
            rc = launch_contract_rows(psi, x, x_dtype, xk, B, Ci, row0, nr, st);
            int np = rc == DISCO_OK ? grad_w_slab(xk, DISCO_F32, gy, gy_dtype, partial, B, Ci, Co,
                                                  groups, K, D.nlat_out, D.nlon_out, row0, nr, L, st)
                                    : rc;
            if (np < 0) {
                rc = np;
                break;
            }
            rc = reduce_into(partial, gw, ngw, np, sidx > 0, st);
            if (rc != DISCO_OK) break;
        }
        if (gx) {
            rc = grad_xk_any(gy, gy_dtype, w, w_dtype, gxk, DISCO_F32, B, Ci, Co, groups, K,
                             D.nlat_out, D.nlon_out, row0, nr, st);
            if (rc == DISCO_OK)
                rc = contract_t_any(psi, gxk, DISCO_F32, gx, gx_dtype, B, Ci, row0, nr, sidx > 0, st);
        }
    }
    hipError_t fe = own_ws ? hipFreeAsync(ws, st) : hipSuccess;
    if (rc != DISCO_OK) return rc;
    if (fe != hipSuccess) {
        (void)hipGetLastError();
        return set_error(DISCO_EHIP, "hipFreeAsync failed: %s", hipGetErrorString(fe));
    }
    return DISCO_OK;
}

}  // namespace disco
