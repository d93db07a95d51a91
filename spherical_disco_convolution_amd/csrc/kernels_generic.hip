// Vector-ALU kernels of the DISCO forward pass (gfx950, wave64):
//  * contract_kernel   - the sparse contraction into the K-expanded tensor
//  * einsum_valu       - channel/basis contraction for any dtype and groups
//  * fused_generic     - contraction and channel/basis contraction in one
//                        kernel, the K-expanded tile kept in LDS
//  * fused_depthwise   - fused pass for one input channel per group, with the
//                        weights folded into the filter taps per channel
//
// Forward equation and Psi: torch_harmonics.DiscreteContinuousConvS2 page.
// The p-shift symmetry of that page lets one row of taps per output latitude
// serve all output longitudes: output q of row j reads input longitudes
// (q*s + p_lo + t) mod nlon_in, t in [0, width), of each window.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "disco_internal.h"
#include "kernels_common.h"

namespace disco {

namespace {

constexpr int kThreads = 256;

// --------------------------------------------------------------------------
// Sparse contraction.  One workgroup per (output row j, channel c, batch b).
// Each window's input row is staged in LDS already rolled to the window start
// (ext[u] = x[(q0*s + p_lo + u) mod nlon_in]), so that lane q reads
// ext[q*s + t]: consecutive lanes read consecutive (s = 1) or stride-s LDS
// words, and the taps are wave-uniform scalar loads.
// --------------------------------------------------------------------------
template <typename TX, typename TO, int KP, int QR>
__global__ __launch_bounds__(kThreads) void contract_kernel(
    const TX* __restrict__ x, TO* __restrict__ xk, const int32_t* __restrict__ win_ptr,
    const DevWindow* __restrict__ wins, const float* __restrict__ vals, int C, int K, int nlat_in,
    int nlon_in, int nlon_out, int s, int row0, int nrows) {
    // output rows row0 .. row0 + nrows - 1 into xk [B, C, K, nrows, nlon_out]
    extern __shared__ float ext[];
    const int j = row0 + blockIdx.x;
    const int c = blockIdx.y;
    const int b = blockIdx.z;
    const TX* xc = x + (size_t)(b * C + c) * nlat_in * nlon_in;
    const int w0 = win_ptr[j], w1 = win_ptr[j + 1];
    const size_t plane = (size_t)nrows * nlon_out;
    TO* out = xk + (size_t)(b * C + c) * K * plane + (size_t)blockIdx.x * nlon_out;

    for (int q0 = 0; q0 < nlon_out; q0 += kThreads * QR) {
        float acc[QR][KP];
#pragma unroll
        for (int r = 0; r < QR; ++r)
#pragma unroll
            for (int k = 0; k < KP; ++k) acc[r][k] = 0.0f;
        for (int wi = w0; wi < w1; ++wi) {
            const DevWindow wd = wins[wi];
            const int len = s * (kThreads * QR - 1) + wd.width;
            const TX* row = xc + (size_t)wd.lat * nlon_in;
            const int start = (int)(((int64_t)q0 * s + wd.p_lo) % nlon_in);
            __syncthreads();
            for (int u = threadIdx.x; u < len; u += kThreads) {
                int p = start + u;
                p -= (p / nlon_in) * nlon_in;
                ext[u] = load_f(row, p);
            }
            __syncthreads();
            const float* v = vals + (size_t)wd.val_off * KP;
            for (int t = 0; t < wd.width; ++t) {
                float vk[KP];
#pragma unroll
                for (int k = 0; k < KP; ++k) vk[k] = v[t * KP + k];
#pragma unroll
                for (int r = 0; r < QR; ++r) {
                    const float xv = ext[(threadIdx.x + kThreads * r) * s + t];
#pragma unroll
                    for (int k = 0; k < KP; ++k) acc[r][k] = fmaf(vk[k], xv, acc[r][k]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < QR; ++r) {
            const int q = q0 + threadIdx.x + kThreads * r;
            if (q < nlon_out) {
#pragma unroll
                for (int k = 0; k < KP; ++k)
                    if (k < K) store_f(out, (size_t)k * plane + q, acc[r][k]);
            }
        }
    }
}

// --------------------------------------------------------------------------
// Channel/basis contraction on the vector ALUs.  Thread = output point n of
// one batch; COT output channels of one group per workgroup row.  Weights are
// wave-uniform (scalar loads), xk rows are read coalesced along n.
// --------------------------------------------------------------------------
template <typename TI, typename TY, int COT>
__global__ __launch_bounds__(kThreads) void einsum_valu(const TI* __restrict__ xk,
                                                          const TI* __restrict__ w,
                                                          const float* __restrict__ bias,
                                                          TY* __restrict__ y, int Ci, int Co,
                                                          int groups, int K, int HW) {
    const int n = blockIdx.x * kThreads + threadIdx.x;
    const int co0 = blockIdx.y * COT;
    const int b = blockIdx.z;
    const int cog = Co / groups, cig = Ci / groups;
    const int grp = co0 / cog;
    if (n >= HW) return;
    float acc[COT];
#pragma unroll
    for (int c = 0; c < COT; ++c) acc[c] = 0.0f;
    const TI* xb = xk + ((size_t)b * Ci + (size_t)grp * cig) * K * HW + n;
    const TI* wr = w + (size_t)co0 * cig * K;
    const int kd = cig * K;
    for (int kk = 0; kk < kd; ++kk) {
        const float xv = load_f(xb, (size_t)kk * HW);
#pragma unroll
        for (int c = 0; c < COT; ++c) acc[c] = fmaf(load_f(wr, (size_t)c * kd + kk), xv, acc[c]);
    }
#pragma unroll
    for (int c = 0; c < COT; ++c) {
        const float bv = bias ? bias[co0 + c] : 0.0f;
        store_f(y, ((size_t)b * Co + co0 + c) * HW + n, acc[c] + bv);
    }
}

// --------------------------------------------------------------------------
// Fused forward, any dtype and groups.  One workgroup per (q tile, output row
// j, batch * group).  Phase 1 builds the K-expanded tile xt[ci][k][q] of the
// group in LDS; phase 2 contracts it with the weights.  The tile never
// reaches device memory.
// --------------------------------------------------------------------------
template <typename T, typename TY, int KP>
__global__ __launch_bounds__(kThreads) void fused_generic(
    const T* __restrict__ x, const T* __restrict__ w, const float* __restrict__ bias,
    TY* __restrict__ y, const int32_t* __restrict__ win_ptr, const DevWindow* __restrict__ wins,
    const float* __restrict__ vals, int Ci, int Co, int groups, int K, int nlat_in, int nlon_in,
    int nlat_out, int nlon_out, int s, int QT, int TC, int seg) {
    extern __shared__ float smem[];
    float* xt = smem;                          // [cig][KP][QT]: X_K of the tile
    float* xs = smem + (size_t)(Ci / groups) * KP * QT;   // [nslot][seg]: staged samples
    const int q0 = blockIdx.x * QT;
    const int j = blockIdx.y;
    const int bg = blockIdx.z;
    const int b = bg / groups, grp = bg % groups;
    const int cig = Ci / groups, cog = Co / groups;
    const int w0 = win_ptr[j], w1 = win_ptr[j + 1];
    const int ql = threadIdx.x % QT;
    const int slot = threadIdx.x / QT;
    const int nslot = kThreads / QT;
    const int q = q0 + ql;
    const bool qvalid = q < nlon_out;
    const T* xg = x + ((size_t)b * Ci + (size_t)grp * cig) * nlat_in * nlon_in;
    // channels c0 + slot for c0 = 0, nslot, ...: per window and chunk of at
    // most TC taps t0 .. t0 + tw - 1, the nslot channels' samples
    // q0 s + p_lo + t0 .. + (QT - 1) s + tw - 1 (mod nlon_in) are staged in LDS
    // once, then each thread runs those taps from there.  The chunking keeps
    // the staging buffer independent of the widest window (polar rows of fine
    // grids span the whole ring).
    for (int c0 = 0; c0 < cig; c0 += nslot) {
        const int ci = c0 + slot;
        float acc[KP];
#pragma unroll
        for (int k = 0; k < KP; ++k) acc[k] = 0.0f;
        for (int wi = w0; wi < w1; ++wi) {
            const DevWindow wd = wins[wi];
            for (int t0 = 0; t0 < wd.width; t0 += TC) {
                const int tw = min(TC, wd.width - t0);
                const int len = (QT - 1) * s + tw;   // <= seg
                const int start = (int)(((int64_t)q0 * s + wd.p_lo + t0) % nlon_in);
                __syncthreads();   // the previous chunk's samples are used
                for (int u = threadIdx.x; u < nslot * len; u += kThreads) {
                    const int cc = u / len, uu = u - cc * len;
                    if (c0 + cc < cig) {
                        int p = start + uu;
                        p -= (p / nlon_in) * nlon_in;
                        xs[cc * seg + uu] =
                            load_f(xg + ((size_t)(c0 + cc) * nlat_in + wd.lat) * nlon_in, p);
                    }
                }
                __syncthreads();
                if (ci < cig && qvalid) {
                    const float* v = vals + ((size_t)wd.val_off + t0) * KP;
                    const float* xr = xs + slot * seg + ql * s;
                    for (int t = 0; t < tw; ++t) {
                        const float xv = xr[t];
#pragma unroll
                        for (int k = 0; k < KP; ++k) acc[k] = fmaf(v[t * KP + k], xv, acc[k]);
                    }
                }
            }
        }
        if (ci < cig) {
#pragma unroll
            for (int k = 0; k < KP; ++k) xt[((size_t)ci * KP + k) * QT + ql] = acc[k];
        }
    }
    __syncthreads();
    if (!qvalid) return;
    for (int co = slot; co < cog; co += nslot) {
        const T* wr = w + ((size_t)grp * cog + co) * cig * K;
        float acc = 0.0f;
        for (int ci = 0; ci < cig; ++ci)
            for (int k = 0; k < K; ++k)
                acc = fmaf(load_f(wr, (size_t)ci * K + k), xt[((size_t)ci * KP + k) * QT + ql], acc);
        const int oc = grp * cog + co;
        if (bias) acc += bias[oc];
        store_f(y, (((size_t)b * Co + oc) * nlat_out + j) * nlon_out + q, acc);
    }
}

// --------------------------------------------------------------------------
// Fused forward for one input channel per group.  Then
//   y[b,co,j,q] = sum_(window, t) (sum_k w[co,0,k] * tap[t][k]) * x[b, grp, lat, q*s + p_lo + t]
// so the weights are folded into the taps once per (co, window) and the inner
// loop is one multiply-add per tap.  One workgroup per (row j, co, batch).
// --------------------------------------------------------------------------
template <typename T, typename TY, int KP, int QR>
__global__ __launch_bounds__(kThreads) void fused_depthwise(
    const T* __restrict__ x, const T* __restrict__ w, const float* __restrict__ bias,
    TY* __restrict__ y, const int32_t* __restrict__ win_ptr, const DevWindow* __restrict__ wins,
    const float* __restrict__ vals, int Ci, int Co, int groups, int K, int nlat_in, int nlon_in,
    int nlat_out, int nlon_out, int s, int max_width) {
    extern __shared__ float smem[];
    float* folded = smem;                       // [max_width]
    float* ext = smem + max_width;              // [s*(256*QR-1) + max_width]
    const int j = blockIdx.x;
    const int co = blockIdx.y;
    const int b = blockIdx.z;
    const int cog = Co / groups;
    const int grp = co / cog;                   // Ci / groups == 1: input channel = grp
    const T* xc = x + ((size_t)b * Ci + grp) * nlat_in * nlon_in;
    float wk[KP];
#pragma unroll
    for (int k = 0; k < KP; ++k) wk[k] = k < K ? load_f(w, (size_t)co * K + k) : 0.0f;
    const int w0 = win_ptr[j], w1 = win_ptr[j + 1];
    TY* out = y + (((size_t)b * Co + co) * nlat_out + j) * nlon_out;
    const float bv = bias ? bias[co] : 0.0f;

    for (int q0 = 0; q0 < nlon_out; q0 += kThreads * QR) {
        float acc[QR];
#pragma unroll
        for (int r = 0; r < QR; ++r) acc[r] = 0.0f;
        for (int wi = w0; wi < w1; ++wi) {
            const DevWindow wd = wins[wi];
            const int len = s * (kThreads * QR - 1) + wd.width;
            const T* row = xc + (size_t)wd.lat * nlon_in;
            const int start = (int)(((int64_t)q0 * s + wd.p_lo) % nlon_in);
            __syncthreads();
            const float* v = vals + (size_t)wd.val_off * KP;
            for (int t = threadIdx.x; t < wd.width; t += kThreads) {
                float f = 0.0f;
#pragma unroll
                for (int k = 0; k < KP; ++k) f = fmaf(wk[k], v[t * KP + k], f);
                folded[t] = f;
            }
            for (int u = threadIdx.x; u < len; u += kThreads) {
                int p = start + u;
                p -= (p / nlon_in) * nlon_in;
                ext[u] = load_f(row, p);
            }
            __syncthreads();
            for (int t = 0; t < wd.width; ++t) {
                const float f = folded[t];
#pragma unroll
                for (int r = 0; r < QR; ++r)
                    acc[r] = fmaf(f, ext[(threadIdx.x + kThreads * r) * s + t], acc[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < QR; ++r) {
            const int q = q0 + threadIdx.x + kThreads * r;
            if (q < nlon_out) store_f(out, q, acc[r] + bv);
        }
    }
}

// The same sum with register tiling, for strides S = 1 and 2.  Thread tid
// owns the QR (4, 6 or 8) consecutive outputs q0 + QR tid + r.  The samples of
// a window's input row are staged in LDS from its first longitude on; for
// stride 2 they are split by parity (even offsets in ext_e, odd in ext_o), so
// that tap t = 2 u + p of output q reads ext_p[(q - q0) + u]: a run of
// consecutive words per thread.  Per chunk of DT taps (32, then 8 for the
// rest of the window) a thread reads its run with 16-byte LDS loads (8-byte
// for QR = 6: lanes 16 or 24 bytes apart, free of bank conflicts) and the
// chunk's folded taps as 16-byte broadcasts, then does QR DT multiply-adds
// from registers.  Windows are padded to a multiple of 8 taps with zero taps
// (the samples they meet are real, finite inputs).  Workgroups take (batch,
// channel, output row) tasks in eight bands, band = workgroup index mod 8
// (workgroups are dispatched to the accelerator dies round-robin): a band is
// a range of (batch, channel) planes walked row by row, so the workgroups in
// flight on a die share each row's Psi values and their planes' input rows in
// its L2.
constexpr int kDwT = 32;     // taps per main register chunk
constexpr int kDwTail = 8;   // taps per chunk past the last full main chunk
constexpr int kDwBands = 8;  // accelerator dies (L2 domains)

// LDS words of one parity array (S = 2) or of the one sample array (S = 1)
// for NT threads of QR outputs and windows padded to wpad taps: the last
// chunk's runs end at QR NT + wpad / S - 1.  The odd array starts 16 banks
// past a 32-word boundary after the even one.
__host__ __device__ constexpr int dw_ext_words(int nt, int qr, int wpad, int s) {
    return qr * nt + wpad / s;
}
__host__ __device__ constexpr int dw_odd_offset(int nt, int qr, int wpad) {
    return (dw_ext_words(nt, qr, wpad, 2) + 31) / 32 * 32 + 16;
}

// One chunk of DT taps starting at t0 for the thread's QR outputs (own is
// the first output's offset within the pass): acc[r] += sum_t tap[t0 + t] *
// sample(own + r, t0 + t).  R = DT / S + QR words per array are read, in
// loads of V words.
template <int DT, int QR, int S>
__device__ __forceinline__ void dw_chunk(const float* __restrict__ folded,
                                         const float* __restrict__ ext_e,
                                         const float* __restrict__ ext_o, int own, int t0,
                                         float (&acc)[QR]) {
    constexpr int V = QR == 6 ? 2 : 4;
    constexpr int R = DT / S + QR;
    static_assert(R % V == 0, "whole loads");
    float tap[DT];
#pragma unroll
    for (int i = 0; i < DT / 4; ++i) {
        const float4 f4 = *reinterpret_cast<const float4*>(folded + t0 + 4 * i);
        tap[4 * i] = f4.x;
        tap[4 * i + 1] = f4.y;
        tap[4 * i + 2] = f4.z;
        tap[4 * i + 3] = f4.w;
    }
    auto load_run = [&](const float* src, float (&e)[R]) {
#pragma unroll
        for (int i = 0; i < R / V; ++i) {
            if constexpr (V == 4) {
                const float4 a = *reinterpret_cast<const float4*>(src + 4 * i);
                e[4 * i] = a.x;
                e[4 * i + 1] = a.y;
                e[4 * i + 2] = a.z;
                e[4 * i + 3] = a.w;
            } else {
                const float2 a = *reinterpret_cast<const float2*>(src + 2 * i);
                e[2 * i] = a.x;
                e[2 * i + 1] = a.y;
            }
        }
    };
    if constexpr (S == 2) {
        // output own + r, tap t0 + 2 u + p: ext_p[own + t0 / 2 + r + u]
        float ee[R], eo[R];
        load_run(ext_e + own + t0 / 2, ee);
        load_run(ext_o + own + t0 / 2, eo);
#pragma unroll
        for (int u = 0; u < DT / 2; ++u)
#pragma unroll
            for (int r = 0; r < QR; ++r) {
                acc[r] = fmaf(tap[2 * u], ee[r + u], acc[r]);
                acc[r] = fmaf(tap[2 * u + 1], eo[r + u], acc[r]);
            }
    } else {
        // output own + r, tap t0 + t: ext[own + t0 + r + t]
        float e[R];
        load_run(ext_e + own + t0, e);
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < QR; ++r) acc[r] = fmaf(tap[t], e[r + t], acc[r]);
    }
}

template <typename T, typename TY, int KP, int QR, int S>
__global__ __launch_bounds__(kThreads) void fused_depthwise_tiled(
    const T* __restrict__ x, const T* __restrict__ w, const float* __restrict__ bias,
    TY* __restrict__ y, const int32_t* __restrict__ win_ptr, const DevWindow* __restrict__ wins,
    const float* __restrict__ vals, int Ci, int Co, int groups, int K, int nlat_in, int nlon_in,
    int nlat_out, int nlon_out, int wpad, int ntasks) {
    extern __shared__ __attribute__((aligned(16))) float smem[];
    const int NT = blockDim.x;
    // task -> (plane = b Co + co, output row j); the whole workgroup returns
    // together past the end (uniform)
    const int band = (int)(blockIdx.x % kDwBands), slot = (int)(blockIdx.x / kDwBands);
    int plane, j;
    const int nplanes = ntasks / nlat_out;
    if (nplanes >= kDwBands) {
        // band = a contiguous range of planes, walked row-major: consecutive
        // workgroups share the row's Psi values, and the band's planes' input
        // rows stay in the die's L2 from one row to the next
        const int p0 = (int)((int64_t)band * nplanes / kDwBands);
        const int np = (int)((int64_t)(band + 1) * nplanes / kDwBands) - p0;
        if (slot >= np * nlat_out) return;
        j = slot / np;
        plane = p0 + slot - j * np;
    } else {
        // few planes: contiguous ranges of the flattened (plane, row) tasks
        const int per = (ntasks + kDwBands - 1) / kDwBands;
        const int task = band * per + slot;
        if (slot >= per || task >= ntasks) return;
        j = task % nlat_out;
        plane = task / nlat_out;
    }
    const int co = plane % Co;
    const int b = plane / Co;
    float* folded = smem;                                  // [wpad]
    float* ext_e = smem + wpad;                            // S = 1: the samples in order
    float* ext_o = ext_e + dw_odd_offset(NT, QR, wpad);    // S = 2 only
    const int cog = Co / groups;
    const int grp = co / cog;
    const T* xc = x + ((size_t)b * Ci + grp) * nlat_in * nlon_in;
    float wk[KP];
#pragma unroll
    for (int k = 0; k < KP; ++k) wk[k] = k < K ? load_f(w, (size_t)co * K + k) : 0.0f;
    const int w0 = win_ptr[j], w1 = win_ptr[j + 1];
    TY* out = y + (((size_t)b * Co + co) * nlat_out + j) * nlon_out;
    const float bv = bias ? bias[co] : 0.0f;
    const int tid = threadIdx.x;
    const int own = QR * tid;   // first of this thread's outputs within a pass
    const int adv = (4 * NT) % nlon_in;   // staging stride of one thread, reduced

    for (int q0 = 0; q0 < nlon_out; q0 += QR * NT) {
        float acc[QR];
#pragma unroll
        for (int r = 0; r < QR; ++r) acc[r] = 0.0f;
        for (int wi = w0; wi < w1; ++wi) {
            const DevWindow wd = wins[wi];
            const int wp = (wd.width + kDwTail - 1) / kDwTail * kDwTail;
            const T* row = xc + (size_t)wd.lat * nlon_in;
            const int start = (int)(((int64_t)q0 * S + wd.p_lo) % nlon_in);
            __syncthreads();   // the previous window's reads are done
            const float* v = vals + (size_t)wd.val_off * KP;
            for (int t = tid; t < wp; t += NT) {
                float f = 0.0f;
                if (t < wd.width) {
#pragma unroll
                    for (int k = 0; k < KP; ++k) f = fmaf(wk[k], v[t * KP + k], f);
                }
                folded[t] = f;
            }
            // samples start + u (mod nlon_in) for the u this window's chunks
            // read (S (QR NT + wp / S) of them, a multiple of 4), four per
            // lane and step: for stride 2 samples u, u + 2 go to ext_e and
            // u + 1, u + 3 to ext_o as 8-byte stores, for stride 1 all four
            // as one 16-byte store
            const int nunits = S * dw_ext_words(NT, QR, wp, S) / 4;
            // this thread's first sample, reduced mod nlon_in once; each later
            // unit advances it by adv < nlon_in, so one conditional
            // subtraction keeps it reduced
            int p0 = start + 4 * tid;
            while (p0 >= nlon_in) p0 -= nlon_in;
            for (int g = tid; g < nunits; g += NT) {
                float v[4];
                if (p0 + 3 < nlon_in) {
                    const T* src = row + p0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = load_f(src, e);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        int p = p0 + e;
                        while (p >= nlon_in) p -= nlon_in;   // rows shorter than 4 wrap more than once
                        v[e] = load_f(row, p);
                    }
                }
                if constexpr (S == 2) {
                    *reinterpret_cast<float2*>(ext_e + 2 * g) = make_float2(v[0], v[2]);
                    *reinterpret_cast<float2*>(ext_o + 2 * g) = make_float2(v[1], v[3]);
                } else {
                    *reinterpret_cast<float4*>(ext_e + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
                }
                p0 += adv;
                if (p0 >= nlon_in) p0 -= nlon_in;
            }
            __syncthreads();
            int t0 = 0;
            for (; t0 + kDwT <= wp; t0 += kDwT)
                dw_chunk<kDwT, QR, S>(folded, ext_e, ext_o, own, t0, acc);
            for (; t0 < wp; t0 += kDwTail)
                dw_chunk<kDwTail, QR, S>(folded, ext_e, ext_o, own, t0, acc);
        }
#pragma unroll
        for (int r = 0; r < QR; ++r) {
            const int q = q0 + own + r;
            if (q < nlon_out) store_f(out, q, acc[r] + bv);
        }
    }
}

int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return set_error(DISCO_EHIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return DISCO_OK;
}

int pick_qr(int nlon_out) {
    int qr = (nlon_out + kThreads - 1) / kThreads;
    // every value returned here has a case in each switch that uses it
    return qr <= 1 ? 1 : qr <= 2 ? 2 : qr <= 3 ? 3 : qr <= 4 ? 4 : qr <= 6 ? 6 : 8;
}

template <typename TX, typename TO, int KP>
int contract_kp(const disco_psi* psi, const void* x, void* xk, int B, int C, int row0, int nrows,
                hipStream_t st) {
    const HostPsi& h = psi->host;
    const DevPsi& d = psi->dev;
    const disco_psi_desc& D = h.desc;
    const int QR = pick_qr(D.nlon_out);
    const size_t lds = (size_t)(h.stride * (kThreads * QR - 1) + d.max_width) * sizeof(float);
    if (lds > 64 * 1024) return set_error(DISCO_EUNSUPPORTED, "row too long for the contraction kernel");
    dim3 grid(nrows, C, B);
#define DISCO_CONTRACT_LAUNCH(Q)                                                                  \
    hipLaunchKernelGGL((contract_kernel<TX, TO, KP, Q>), grid, dim3(kThreads), lds, st,           \
                       (const TX*)x, (TO*)xk, d.win_ptr, d.windows, d.vals, C, h.K, D.nlat_in,    \
                       D.nlon_in, D.nlon_out, h.stride, row0, nrows)
    KernelTimer timer("contract_kernel", st);
    switch (QR) {
        case 1: DISCO_CONTRACT_LAUNCH(1); break;
        case 2: DISCO_CONTRACT_LAUNCH(2); break;
        case 3: DISCO_CONTRACT_LAUNCH(3); break;
        case 4: DISCO_CONTRACT_LAUNCH(4); break;
        case 6: DISCO_CONTRACT_LAUNCH(6); break;
        default: DISCO_CONTRACT_LAUNCH(8); break;
    }
#undef DISCO_CONTRACT_LAUNCH
    return check_launch("contract");
}

template <typename TX, typename TO>
int contract_dispatch(const disco_psi* psi, const void* x, void* xk, int B, int C, hipStream_t st,
                      int row0 = 0, int nrows = -1) {
    if (nrows < 0) nrows = psi->host.desc.nlat_out;
    switch (psi->dev.KP) {
#define DISCO_CK(N) \
    case N: return contract_kp<TX, TO, N>(psi, x, xk, B, C, row0, nrows, st);
        DISCO_CK(1) DISCO_CK(2) DISCO_CK(4) DISCO_CK(8) DISCO_CK(12) DISCO_CK(16) DISCO_CK(20)
        DISCO_CK(24) DISCO_CK(28) DISCO_CK(32)
#undef DISCO_CK
        default: return set_error(DISCO_EUNSUPPORTED, "K = %d is not supported by the contraction "
                                  "kernel (K <= 32)", psi->host.K);
    }
}

}  // namespace

int launch_contract(const disco_psi* psi, const void* x, int x_dtype, void* xk, int xk_dtype,
                    int B, int C, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    int rc = DISCO_OK;
    if (x_dtype == DISCO_BF16 && xk_dtype == DISCO_BF16 &&
        try_launch_contract_mfma(psi, x, xk, B, C, st, &rc))
        return rc;
    if (x_dtype == DISCO_F32 && xk_dtype == DISCO_F32)
        return contract_dispatch<float, float>(psi, x, xk, B, C, st);
    if (x_dtype == DISCO_F32 && xk_dtype == DISCO_BF16)
        return contract_dispatch<float, bf16_t>(psi, x, xk, B, C, st);
    if (x_dtype == DISCO_BF16 && xk_dtype == DISCO_F32)
        return contract_dispatch<bf16_t, float>(psi, x, xk, B, C, st);
    return contract_dispatch<bf16_t, bf16_t>(psi, x, xk, B, C, st);
}

// The contraction of output rows row0 .. row0 + nrows - 1 into a float32
// [B, C, K, nrows, nlon_out] tensor (the fused backward's recomputed X_K).
int launch_contract_rows(const disco_psi* psi, const void* x, int x_dtype, float* xk, int B, int C,
                         int row0, int nrows, hipStream_t st) {
    if (x_dtype == DISCO_F32)
        return contract_dispatch<float, float>(psi, x, xk, B, C, st, row0, nrows);
    return contract_dispatch<bf16_t, float>(psi, x, xk, B, C, st, row0, nrows);
}

// defined in kernels_einsum_mfma.hip
int launch_einsum_mfma_bf16(const void* xk, const void* w, const float* bias, void* y, int y_dtype,
                            int B, int Ci, int Co, int groups, int K, int HW, hipStream_t st);

namespace {
template <typename TI, typename TY>
int einsum_valu_launch(const void* xk, const void* w, const float* bias, void* y, int B, int Ci,
                       int Co, int groups, int K, int HW, hipStream_t st) {
    const int cog = Co / groups;
    int cot = 16;
    while (cog % cot) cot /= 2;
    dim3 grid((HW + kThreads - 1) / kThreads, Co / cot, B);
#define DISCO_EINSUM_LAUNCH(N)                                                                   \
    hipLaunchKernelGGL((einsum_valu<TI, TY, N>), grid, dim3(kThreads), 0, st, (const TI*)xk,     \
                       (const TI*)w, bias, (TY*)y, Ci, Co, groups, K, HW)
    KernelTimer timer("einsum_valu", st);
    switch (cot) {
        case 16: DISCO_EINSUM_LAUNCH(16); break;
        case 8: DISCO_EINSUM_LAUNCH(8); break;
        case 4: DISCO_EINSUM_LAUNCH(4); break;
        case 2: DISCO_EINSUM_LAUNCH(2); break;
        default: DISCO_EINSUM_LAUNCH(1); break;
    }
#undef DISCO_EINSUM_LAUNCH
    return check_launch("einsum");
}
}  // namespace

int launch_einsum(const void* xk, int xk_dtype, const void* w, int w_dtype, const float* bias,
                  void* y, int y_dtype, int B, int Ci, int Co, int groups, int K, int nlat_out,
                  int nlon_out, void* stream) {
    (void)w_dtype;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int HW = nlat_out * nlon_out;
    const int cog = Co / groups, cig = Ci / groups;
    if (xk_dtype == DISCO_BF16 && cog >= 32 && cig * K >= 32)
        return launch_einsum_mfma_bf16(xk, w, bias, y, y_dtype, B, Ci, Co, groups, K, HW, st);
    if (xk_dtype == DISCO_F32)
        return y_dtype == DISCO_F32
                   ? einsum_valu_launch<float, float>(xk, w, bias, y, B, Ci, Co, groups, K, HW, st)
                   : einsum_valu_launch<float, bf16_t>(xk, w, bias, y, B, Ci, Co, groups, K, HW, st);
    return y_dtype == DISCO_F32
               ? einsum_valu_launch<bf16_t, float>(xk, w, bias, y, B, Ci, Co, groups, K, HW, st)
               : einsum_valu_launch<bf16_t, bf16_t>(xk, w, bias, y, B, Ci, Co, groups, K, HW, st);
}

namespace {

template <typename T, typename TY, int KP>
int fused_generic_launch(const disco_psi* psi, const void* x, const void* w, const float* bias,
                         void* y, int B, int Ci, int Co, int groups, hipStream_t st) {
    const HostPsi& h = psi->host;
    const DevPsi& d = psi->dev;
    const disco_psi_desc& D = h.desc;
    const int cig = Ci / groups;
    // output-tile width QT and tap chunk TC: the X_K tile [cig][KP][QT] plus
    // the staged samples [kThreads / QT][(QT - 1) s + TC] within 64 KiB.  QT is
    // at most 256 and no wider than two rows' worth of outputs; TC is the
    // widest window, or less (down to 16) where that does not fit.
    auto lds_of = [&](int qt, int tc) {
        const size_t seg = (size_t)(qt - 1) * h.stride + tc;
        return ((size_t)cig * KP * qt + (size_t)(kThreads / qt) * seg) * sizeof(float);
    };
    const int tc_max = std::max(1, d.max_width);
    int QT = 256;
    while (QT > 8 && QT / 2 >= D.nlon_out) QT /= 2;
    int TC = tc_max;
    // the widest QT whose tile fits with chunks of at least 64 taps (or the
    // whole widest window), then smaller chunks if even QT = 8 does not fit
    for (;;) {
        TC = tc_max;
        while (TC > 64 && lds_of(QT, TC) > 64 * 1024) TC = std::max(64, TC / 2);
        if (lds_of(QT, TC) <= 64 * 1024 || QT <= 8) break;
        QT /= 2;
    }
    while (TC > 16 && lds_of(QT, TC) > 64 * 1024) TC = std::max(16, TC / 2);
    const size_t lds = lds_of(QT, TC);
    if (lds > 64 * 1024)
        return set_error(DISCO_EUNSUPPORTED, "Ci/groups * K too large for the generic fused kernel");
    const int seg = (QT - 1) * h.stride + TC;
    dim3 grid((D.nlon_out + QT - 1) / QT, D.nlat_out, B * groups);
    KernelTimer timer("fused_generic", st);
    hipLaunchKernelGGL((fused_generic<T, TY, KP>), grid, dim3(kThreads), lds, st, (const T*)x,
                       (const T*)w, bias, (TY*)y, d.win_ptr, d.windows, d.vals, Ci, Co, groups,
                       h.K, D.nlat_in, D.nlon_in, D.nlat_out, D.nlon_out, h.stride, QT, TC, seg);
    return check_launch("fused_generic");
}

template <typename T, typename TY, int KP>
int fused_depthwise_launch(const disco_psi* psi, const void* x, const void* w, const float* bias,
                           void* y, int B, int Ci, int Co, int groups, hipStream_t st) {
    const HostPsi& h = psi->host;
    const DevPsi& d = psi->dev;
    const disco_psi_desc& D = h.desc;
    const int QR = pick_qr(D.nlon_out);
    dim3 grid(D.nlat_out, Co, B);
    if (h.stride <= 2) {
        // register-tiled form; LDS holds the padded folded taps and the
        // staged samples (by parity for stride 2).  Outputs per thread: the
        // QR of 4, 6, 8 whose passes leave the fewest idle outputs (the
        // smaller on ties: at 720 outputs, 4 per thread with three waves
        // timed 4.37 ms against 4.51 ms for 6 per thread with two, whose runs
        // need 8-byte loads).
        int qr = 4, nt = 64;
        double best = -1.0;
        for (int q : {4, 6, 8}) {
            const int need = (D.nlon_out + q - 1) / q;
            const int t = std::min(kThreads, (need + 63) / 64 * 64);
            const int passes = (D.nlon_out + q * t - 1) / (q * t);
            const double use = (double)D.nlon_out / ((double)passes * q * t);
            if (use > best) {
                best = use;
                qr = q;
                nt = t;
            }
        }
        const int wpad = (d.max_width + kDwTail - 1) / kDwTail * kDwTail;
        const int S = h.stride;
        const size_t words = (size_t)wpad + (S == 2 ? (size_t)dw_odd_offset(nt, qr, wpad) +
                                                          dw_ext_words(nt, qr, wpad, 2)
                                                    : (size_t)dw_ext_words(nt, qr, wpad, 1));
        const size_t tl = words * sizeof(float);
        const int64_t ntasks = (int64_t)B * Co * D.nlat_out;
        if (tl <= 64 * 1024 && ntasks < (int64_t)1 << 31) {
            // workgroups per band: the largest band's tasks (see the kernel)
            const int64_t nplanes = (int64_t)B * Co;
            const int64_t per = nplanes >= kDwBands
                                    ? (nplanes + kDwBands - 1) / kDwBands * D.nlat_out
                                    : (ntasks + kDwBands - 1) / kDwBands;
            const dim3 tgrid((unsigned)(per * kDwBands));
            KernelTimer timer("fused_depthwise", st);
#define DISCO_DWT(Q, SS)                                                                          \
    hipLaunchKernelGGL((fused_depthwise_tiled<T, TY, KP, Q, SS>), tgrid, dim3(nt), tl, st,        \
                       (const T*)x, (const T*)w, bias, (TY*)y, d.win_ptr, d.windows, d.vals, Ci,  \
                       Co, groups, h.K, D.nlat_in, D.nlon_in, D.nlat_out, D.nlon_out, wpad,       \
                       (int)ntasks)
#define DISCO_DWT_S(Q)   \
    if (S == 1) {        \
        DISCO_DWT(Q, 1); \
    } else {             \
        DISCO_DWT(Q, 2); \
    }
            if (qr == 4) {
                DISCO_DWT_S(4)
            } else if (qr == 6) {
                DISCO_DWT_S(6)
            } else {
                DISCO_DWT_S(8)
            }
#undef DISCO_DWT_S
#undef DISCO_DWT
            return check_launch("fused_depthwise");
        }
    }
    const size_t lds =
        (size_t)(d.max_width + h.stride * (kThreads * QR - 1) + d.max_width) * sizeof(float);
    if (lds > 64 * 1024) return set_error(DISCO_EUNSUPPORTED, "row too long for the depthwise kernel");
#define DISCO_DW_LAUNCH(Q)                                                                       \
    hipLaunchKernelGGL((fused_depthwise<T, TY, KP, Q>), grid, dim3(kThreads), lds, st,          \
                       (const T*)x, (const T*)w, bias, (TY*)y, d.win_ptr, d.windows, d.vals, Ci, \
                       Co, groups, h.K, D.nlat_in, D.nlon_in, D.nlat_out, D.nlon_out, h.stride,  \
                       d.max_width)
    KernelTimer timer("fused_depthwise", st);
    switch (QR) {
        case 1: DISCO_DW_LAUNCH(1); break;
        case 2: DISCO_DW_LAUNCH(2); break;
        case 3: DISCO_DW_LAUNCH(3); break;
        case 4: DISCO_DW_LAUNCH(4); break;
        case 6: DISCO_DW_LAUNCH(6); break;
        default: DISCO_DW_LAUNCH(8); break;
    }
#undef DISCO_DW_LAUNCH
    return check_launch("fused_depthwise");
}

template <typename T, typename TY>
int fused_vector(const disco_psi* psi, const void* x, const void* w, const float* bias, void* y,
                 int B, int Ci, int Co, int groups, hipStream_t st) {
    const bool dw = (Ci / groups) == 1;
#define DISCO_FUSED_KP(N)                                                                  \
    return dw ? fused_depthwise_launch<T, TY, N>(psi, x, w, bias, y, B, Ci, Co, groups, st) \
              : fused_generic_launch<T, TY, N>(psi, x, w, bias, y, B, Ci, Co, groups, st)
    switch (psi->dev.KP) {
        case 1: DISCO_FUSED_KP(1);
        case 2: DISCO_FUSED_KP(2);
        case 4: DISCO_FUSED_KP(4);
        case 8: DISCO_FUSED_KP(8);
        case 12: DISCO_FUSED_KP(12);
        case 16: DISCO_FUSED_KP(16);
        case 20: DISCO_FUSED_KP(20);
        case 24: DISCO_FUSED_KP(24);
        case 28: DISCO_FUSED_KP(28);
        case 32: DISCO_FUSED_KP(32);
        default:
            return set_error(DISCO_EUNSUPPORTED, "K = %d is not supported by the fused kernels "
                             "(K <= 32)", psi->host.K);
    }
#undef DISCO_FUSED_KP
}

}  // namespace

// defined in kernels_fused_mfma.hip; returns 1 if it handled the call.  With
// frag_ws non-NULL the weight fragments go there (frag_ws_bytes available)
// instead of stream-ordered workspace.
int try_launch_fused_mfma(const disco_psi* psi, const void* x, const void* w, const float* bias,
                          void* y, int y_dtype, int B, int Ci, int Co, int groups, hipStream_t st,
                          int* rc, void* frag_ws, size_t frag_ws_bytes);
int noalloc_scratch(void** ptr, size_t* bytes);

// defined in kernels_spectral.hip; each returns 1 if it handled the call
int try_launch_fused_spectral(const disco_psi* psi, const void* x, const void* w,
                              const float* bias, void* y, int y_dtype, int B, int Ci, int Co,
                              int groups, hipStream_t st, int* rc);
int try_launch_fused_spectral32(const disco_psi* psi, const void* x, const void* w,
                                const float* bias, void* y, int y_dtype, int B, int Ci, int Co,
                                int groups, hipStream_t st, int* rc);

namespace {
// The direct algorithms: the matrix-core kernel for the bf16 layers it takes,
// the vector kernels otherwise.
int launch_fused_direct(const disco_psi* psi, const void* x, int dtype, const void* w,
                        const float* bias, void* y, int y_dtype, int B, int Ci, int Co, int groups,
                        hipStream_t st, void* frag_ws, size_t frag_ws_bytes) {
    int rc = DISCO_OK;
    if (dtype == DISCO_BF16 && try_launch_fused_mfma(psi, x, w, bias, y, y_dtype, B, Ci, Co,
                                                     groups, st, &rc, frag_ws, frag_ws_bytes))
        return rc;
    if (dtype == DISCO_F32)
        return y_dtype == DISCO_F32
                   ? fused_vector<float, float>(psi, x, w, bias, y, B, Ci, Co, groups, st)
                   : fused_vector<float, bf16_t>(psi, x, w, bias, y, B, Ci, Co, groups, st);
    return y_dtype == DISCO_F32
               ? fused_vector<bf16_t, float>(psi, x, w, bias, y, B, Ci, Co, groups, st)
               : fused_vector<bf16_t, bf16_t>(psi, x, w, bias, y, B, Ci, Co, groups, st);
}
}  // namespace

int launch_fused(const disco_psi* psi, const void* x, int dtype, const void* w, const float* bias,
                 void* y, int y_dtype, int B, int Ci, int Co, int groups, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    int rc = DISCO_OK;
    if (dtype == DISCO_BF16 &&
        try_launch_fused_spectral(psi, x, w, bias, y, y_dtype, B, Ci, Co, groups, st, &rc))
        return rc;
    if (dtype == DISCO_F32 &&
        try_launch_fused_spectral32(psi, x, w, bias, y, y_dtype, B, Ci, Co, groups, st, &rc))
        return rc;
    return launch_fused_direct(psi, x, dtype, w, bias, y, y_dtype, B, Ci, Co, groups, st, nullptr,
                               0);
}

int launch_fused_noalloc(const disco_psi* psi, const void* x, int dtype, const void* w,
                         const float* bias, void* y, int y_dtype, int B, int Ci, int Co,
                         int groups, void* stream) {
    void* ws = nullptr;
    size_t bytes = 0;
    int rc = noalloc_scratch(&ws, &bytes);
    if (rc != DISCO_OK) return rc;
    return launch_fused_direct(psi, x, dtype, w, bias, y, y_dtype, B, Ci, Co, groups,
                               static_cast<hipStream_t>(stream), ws, bytes);
}

}  // namespace disco
