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
    int nlon_in, int nlat_out, int nlon_out, int s) {
    extern __shared__ float ext[];
    const int j = blockIdx.x;
    const int c = blockIdx.y;
    const int b = blockIdx.z;
    const TX* xc = x + (size_t)(b * C + c) * nlat_in * nlon_in;
    const int w0 = win_ptr[j], w1 = win_ptr[j + 1];
    const size_t plane = (size_t)nlat_out * nlon_out;
    TO* out = xk + (size_t)(b * C + c) * K * plane + (size_t)j * nlon_out;

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
    int nlat_out, int nlon_out, int s, int QT, int seg) {
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

    // channels c0 + slot for c0 = 0, nslot, ...: per window, the nslot
    // channels' samples q0 s + p_lo .. + (QT - 1) s + width - 1 (mod nlon_in)
    // are staged in LDS once, then each thread runs its taps from there
    for (int c0 = 0; c0 < cig; c0 += nslot) {
        const int ci = c0 + slot;
        float acc[KP];
#pragma unroll
        for (int k = 0; k < KP; ++k) acc[k] = 0.0f;
        for (int wi = w0; wi < w1; ++wi) {
            const DevWindow wd = wins[wi];
            const int len = (QT - 1) * s + wd.width;   // <= seg
            const int start = (int)(((int64_t)q0 * s + wd.p_lo) % nlon_in);
            __syncthreads();   // the previous window's samples are used
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
                const float* v = vals + (size_t)wd.val_off * KP;
                const float* xr = xs + slot * seg + ql * s;
                for (int t = 0; t < wd.width; ++t) {
                    const float xv = xr[t];
#pragma unroll
                    for (int k = 0; k < KP; ++k) acc[k] = fmaf(v[t * KP + k], xv, acc[k]);
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

// The same sum with register tiling, for strides S = 1 and 2: thread tid
// owns the QR consecutive outputs q0 + tid QR + r, whose input samples for
// taps t0 .. t0 + DT - 1 form one run of (QR - 1) S + DT values.  That run is
// read from LDS once per tap chunk and kept in registers; the folded taps are
// LDS broadcasts.  The tap loop is padded to a multiple of DT with zero taps
// (the samples they meet are real, finite inputs).
constexpr int kDwTile = 16;   // taps per register chunk

template <typename T, typename TY, int KP, int QR, int S>
__global__ __launch_bounds__(kThreads) void fused_depthwise_tiled(
    const T* __restrict__ x, const T* __restrict__ w, const float* __restrict__ bias,
    TY* __restrict__ y, const int32_t* __restrict__ win_ptr, const DevWindow* __restrict__ wins,
    const float* __restrict__ vals, int Ci, int Co, int groups, int K, int nlat_in, int nlon_in,
    int nlat_out, int nlon_out, int max_width_padded) {
    constexpr int DT = kDwTile;
    constexpr int NE = (QR - 1) * S + DT;   // samples per chunk
    extern __shared__ float smem[];
    float* folded = smem;                           // [max_width_padded]
    float* ext = smem + max_width_padded;           // [S (kThreads QR - 1) + max_width_padded]
    const int j = blockIdx.x;
    const int co = blockIdx.y;
    const int b = blockIdx.z;
    const int cog = Co / groups;
    const int grp = co / cog;
    const T* xc = x + ((size_t)b * Ci + grp) * nlat_in * nlon_in;
    float wk[KP];
#pragma unroll
    for (int k = 0; k < KP; ++k) wk[k] = k < K ? load_f(w, (size_t)co * K + k) : 0.0f;
    const int w0 = win_ptr[j], w1 = win_ptr[j + 1];
    TY* out = y + (((size_t)b * Co + co) * nlat_out + j) * nlon_out;
    const float bv = bias ? bias[co] : 0.0f;
    const int tbase = threadIdx.x * QR * S;

    for (int q0 = 0; q0 < nlon_out; q0 += kThreads * QR) {
        float acc[QR];
#pragma unroll
        for (int r = 0; r < QR; ++r) acc[r] = 0.0f;
        for (int wi = w0; wi < w1; ++wi) {
            const DevWindow wd = wins[wi];
            const int wpad = (wd.width + DT - 1) / DT * DT;
            const int len = S * (kThreads * QR - 1) + wpad;
            const T* row = xc + (size_t)wd.lat * nlon_in;
            const int start = (int)(((int64_t)q0 * S + wd.p_lo) % nlon_in);
            __syncthreads();
            const float* v = vals + (size_t)wd.val_off * KP;
            for (int t = threadIdx.x; t < wpad; t += kThreads) {
                float f = 0.0f;
                if (t < wd.width) {
#pragma unroll
                    for (int k = 0; k < KP; ++k) f = fmaf(wk[k], v[t * KP + k], f);
                }
                folded[t] = f;
            }
            for (int u = threadIdx.x; u < len; u += kThreads) {
                int p = start + u;
                p -= (p / nlon_in) * nlon_in;
                ext[u] = load_f(row, p);
            }
            __syncthreads();
            for (int t0 = 0; t0 < wpad; t0 += DT) {
                float e[NE];
#pragma unroll
                for (int m = 0; m < NE; ++m) e[m] = ext[tbase + t0 + m];
#pragma unroll
                for (int t = 0; t < DT; ++t) {
                    const float f = folded[t0 + t];
#pragma unroll
                    for (int r = 0; r < QR; ++r) acc[r] = fmaf(f, e[r * S + t], acc[r]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < QR; ++r) {
            const int q = q0 + threadIdx.x * QR + r;
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
int contract_kp(const disco_psi* psi, const void* x, void* xk, int B, int C, hipStream_t st) {
    const HostPsi& h = psi->host;
    const DevPsi& d = psi->dev;
    const disco_psi_desc& D = h.desc;
    const int QR = pick_qr(D.nlon_out);
    const size_t lds = (size_t)(h.stride * (kThreads * QR - 1) + d.max_width) * sizeof(float);
    if (lds > 64 * 1024) return set_error(DISCO_EUNSUPPORTED, "row too long for the contraction kernel");
    dim3 grid(D.nlat_out, C, B);
#define DISCO_CONTRACT_LAUNCH(Q)                                                                  \
    hipLaunchKernelGGL((contract_kernel<TX, TO, KP, Q>), grid, dim3(kThreads), lds, st,           \
                       (const TX*)x, (TO*)xk, d.win_ptr, d.windows, d.vals, C, h.K, D.nlat_in,    \
                       D.nlon_in, D.nlat_out, D.nlon_out, h.stride)
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
int contract_dispatch(const disco_psi* psi, const void* x, void* xk, int B, int C, hipStream_t st) {
    switch (psi->dev.KP) {
        case 1: return contract_kp<TX, TO, 1>(psi, x, xk, B, C, st);
        case 2: return contract_kp<TX, TO, 2>(psi, x, xk, B, C, st);
        case 4: return contract_kp<TX, TO, 4>(psi, x, xk, B, C, st);
        case 8: return contract_kp<TX, TO, 8>(psi, x, xk, B, C, st);
        case 12: return contract_kp<TX, TO, 12>(psi, x, xk, B, C, st);
        case 16: return contract_kp<TX, TO, 16>(psi, x, xk, B, C, st);
        case 20: return contract_kp<TX, TO, 20>(psi, x, xk, B, C, st);
        case 24: return contract_kp<TX, TO, 24>(psi, x, xk, B, C, st);
        case 28: return contract_kp<TX, TO, 28>(psi, x, xk, B, C, st);
        case 32: return contract_kp<TX, TO, 32>(psi, x, xk, B, C, st);
        default: return set_error(DISCO_EUNSUPPORTED, "K = %d is not supported by the contraction "
                                  "kernel (K <= 32)", psi->host.K);
    }
}

}  // namespace

// defined in kernels_fused_mfma.hip: the matrix-core contraction (bf16 x and
// xk); returns 0 when the shape is not one it takes
int try_launch_contract_mfma(const disco_psi* psi, const void* x, void* xk, int B, int C,
                             hipStream_t st, int* rc);

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
    // output-tile width QT: the X_K tile [cig][KP][QT] plus the staged samples
    // [kThreads / QT][(QT - 1) s + max_width] within 64 KiB, at most 256 and
    // no wider than two rows' worth of outputs
    auto lds_of = [&](int qt) {
        const size_t seg = (size_t)(qt - 1) * h.stride + d.max_width;
        return ((size_t)cig * KP * qt + (size_t)(kThreads / qt) * seg) * sizeof(float);
    };
    int QT = 256;
    while (QT > 8 && lds_of(QT) > 64 * 1024) QT /= 2;
    while (QT > 8 && QT / 2 >= D.nlon_out) QT /= 2;
    const size_t lds = lds_of(QT);
    if (lds > 64 * 1024)
        return set_error(DISCO_EUNSUPPORTED, "Ci/groups * K too large for the generic fused kernel");
    const int seg = (QT - 1) * h.stride + d.max_width;
    dim3 grid((D.nlon_out + QT - 1) / QT, D.nlat_out, B * groups);
    KernelTimer timer("fused_generic", st);
    hipLaunchKernelGGL((fused_generic<T, TY, KP>), grid, dim3(kThreads), lds, st, (const T*)x,
                       (const T*)w, bias, (TY*)y, d.win_ptr, d.windows, d.vals, Ci, Co, groups,
                       h.K, D.nlat_in, D.nlon_in, D.nlat_out, D.nlon_out, h.stride, QT, seg);
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
        // register-tiled form; LDS holds the padded folded taps and the samples
        const int wpad = (d.max_width + kDwTile - 1) / kDwTile * kDwTile;
        const size_t tl = (size_t)(wpad + h.stride * (kThreads * QR - 1) + wpad) * sizeof(float);
        if (tl <= 64 * 1024) {
#define DISCO_DWT(Q, SS)                                                                          \
    hipLaunchKernelGGL((fused_depthwise_tiled<T, TY, KP, Q, SS>), grid, dim3(kThreads), tl, st,   \
                       (const T*)x, (const T*)w, bias, (TY*)y, d.win_ptr, d.windows, d.vals, Ci,  \
                       Co, groups, h.K, D.nlat_in, D.nlon_in, D.nlat_out, D.nlon_out, wpad)
#define DISCO_DWT_S(Q)             \
    if (h.stride == 1) {           \
        DISCO_DWT(Q, 1);           \
    } else {                       \
        DISCO_DWT(Q, 2);           \
    }
            KernelTimer timer("fused_depthwise", st);
            switch (QR) {
                case 1: DISCO_DWT_S(1) break;
                case 2: DISCO_DWT_S(2) break;
                case 3: DISCO_DWT_S(3) break;
                case 4: DISCO_DWT_S(4) break;
                case 6: DISCO_DWT_S(6) break;
                default: DISCO_DWT_S(8) break;
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

// defined in kernels_fused_mfma.hip; returns 1 if it handled the call
int try_launch_fused_mfma(const disco_psi* psi, const void* x, const void* w, const float* bias,
                          void* y, int y_dtype, int B, int Ci, int Co, int groups, hipStream_t st,
                          int* rc);

// defined in kernels_spectral.hip; returns 1 if it handled the call
int try_launch_fused_spectral(const disco_psi* psi, const void* x, const void* w,
                              const float* bias, void* y, int y_dtype, int B, int Ci, int Co,
                              int groups, hipStream_t st, int* rc);

int launch_fused(const disco_psi* psi, const void* x, int dtype, const void* w, const float* bias,
                 void* y, int y_dtype, int B, int Ci, int Co, int groups, void* stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    int rc = DISCO_OK;
    if (dtype == DISCO_BF16 &&
        try_launch_fused_spectral(psi, x, w, bias, y, y_dtype, B, Ci, Co, groups, st, &rc))
        return rc;
    if (dtype == DISCO_BF16 &&
        try_launch_fused_mfma(psi, x, w, bias, y, y_dtype, B, Ci, Co, groups, st, &rc))
        return rc;
    if (dtype == DISCO_F32)
        return y_dtype == DISCO_F32
                   ? fused_vector<float, float>(psi, x, w, bias, y, B, Ci, Co, groups, st)
                   : fused_vector<float, bf16_t>(psi, x, w, bias, y, B, Ci, Co, groups, st);
    return y_dtype == DISCO_F32
               ? fused_vector<bf16_t, float>(psi, x, w, bias, y, B, Ci, Co, groups, st)
               : fused_vector<bf16_t, bf16_t>(psi, x, w, bias, y, B, Ci, Co, groups, st);
}

}  // namespace disco
