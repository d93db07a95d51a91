// Matrix-core fused forward of the DISCO convolution (bf16 in, float32
// accumulation), gfx950.
//
// What is computed (torch_harmonics.DiscreteContinuousConvS2 page, forward
// equation; `fused` parameter: contraction and weight multiplication without
// storing the K-expanded intermediate):
//
//   xk[ci,k,q] = sum_{windows (i,p_lo,W)} sum_{t<W} Psi[k,t] x[ci, i, (s*q + p_lo + t) mod nlon_in]
//   y[co,q]    = sum_{ci,k} w[co,ci,k] xk[ci,k,q]
//
// for one output row j.  Both sums run on v_mfma_f32_32x32x16_bf16.
//
// Contraction as banded Toeplitz products.  For a block of four consecutive
// outputs q..q+3 and one window, xk over the 32 (qq, k) pairs (qq < 4,
// k < 8; k >= K is zero) and 32 channels is
//     C[(qq,k), ci] = sum_x T[(qq,k), x] * X[x, ci],   T[(qq,k), x] = Psi[k, x - delta - s*qq]
// where x runs over input longitudes from an 8-aligned start and delta (the
// misalignment of the band) takes one of two values per window.  T depends
// only on the window, the alignment class and the 16-wide chunk of x, so it
// is tabulated once on the host in MFMA operand order ("tap fragments"); X is
// read from input rows staged in LDS.  Lanes of the result hold four
// consecutive k of one channel for each qq, which is written to the LDS tile
// xk[q][ci*8 + k] with 8-byte stores.
//
// Channel/basis GEMM: y[co, q] += W[co, kappa] * xk[q][kappa], kappa = ci*8 + k,
// with W pre-tiled into operand fragments by a small preparation kernel.
//
// One workgroup (4 waves) owns one output row and Q output longitudes for all
// output channels.  Work items are distributed over the 8 XCDs in contiguous
// latitude bands of equal cost (the polar rows carry ~100x more taps than the
// equatorial ones), so that workgroups sharing input rows share an L2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>

#include "disco_internal.h"
#include "kernels_common.h"

namespace disco {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kNumXcd = 8;
constexpr int kXsStride = 136;      // staged row length (elements): 128 + 8 pad
constexpr int kXsLen = 128;         // longitudes staged per piece
constexpr int kXkPad = 8;           // xk tile row padding (elements)

struct MfmaWin {
    int32_t lat, p_lo, width, nch0, nch1, tap0, tap1, pad;
};

// Tap fragment values: lane l, element e of chunk c for alignment delta.
inline float tap_value(const HostPsi& h, const Window& wd, int delta, int chunk, int lane, int e) {
    const int m = lane & 31;
    const int qq = m >> 3, k = m & 7;
    const int x = 16 * chunk + 8 * (lane >> 5) + e;
    const int t = x - delta - h.stride * qq;
    if (k >= h.K || t < 0 || t >= wd.width) return 0.0f;
    return (float)h.win_vals[(size_t)(wd.val_off + t) * h.K + k];
}

uint16_t host_bf16(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

}  // namespace

// Layout of `info` (int32): [0] magic, [1] nwin, [2] offset of the MfmaWin array,
// [3] offset of win_ptr, [4] Q, [5] nqt, [6] offset of the work lists, [7] list stride.
enum { kInfoMagic = 0, kInfoNwin, kInfoWins, kInfoWinPtr, kInfoQ, kInfoNqt, kInfoWork,
       kInfoStride, kInfoSize };
constexpr int kQ = 128;   // output longitudes per workgroup

int build_mfma_tables(disco_psi* psi, std::vector<char>& taps, std::vector<int32_t>& info) {
    taps.clear();
    info.clear();
    const HostPsi& h = psi->host;
    const disco_psi_desc& D = h.desc;
    // The matrix-core path covers K <= 8, longitudes a multiple of 8 and
    // strides 1 and 2 (the latter: one alignment class).
    if (h.K > 8 || D.nlon_in % 8 != 0 || h.stride > 2) return DISCO_OK;
    const int S = h.stride;
    const int nwin = (int)h.windows.size();
    std::vector<MfmaWin> wins(nwin);
    size_t nfrag = 0;
    for (int n = 0; n < nwin; ++n) {
        const Window& wd = h.windows[n];
        MfmaWin& m = wins[n];
        m.lat = wd.lat;
        m.p_lo = wd.p_lo;
        m.width = wd.width;
        const int d0 = wd.p_lo & 7;
        m.nch0 = (d0 + 3 * S + wd.width + 15) / 16;
        m.tap0 = (int32_t)nfrag;
        nfrag += m.nch0;
        if (S & 1) {
            const int d1 = (wd.p_lo + 4) & 7;
            m.nch1 = (d1 + 3 * S + wd.width + 15) / 16;
            m.tap1 = (int32_t)nfrag;
            nfrag += m.nch1;
        } else {
            m.nch1 = 0;
            m.tap1 = m.tap0;
        }
        m.pad = 0;
    }
    if (nfrag > (size_t)0x7fffffff / 1024) return DISCO_OK;
    try {
        taps.assign(nfrag * 1024, 0);
    } catch (const std::bad_alloc&) {
        return set_error(DISCO_ENOMEM, "host allocation failed (tap fragments)");
    }
    uint16_t* tp = reinterpret_cast<uint16_t*>(taps.data());
    for (int n = 0; n < nwin; ++n) {
        const Window& wd = h.windows[n];
        const MfmaWin& m = wins[n];
        for (int cls = 0; cls < ((S & 1) ? 2 : 1); ++cls) {
            const int delta = (wd.p_lo + 4 * cls) & 7;
            const int nch = cls ? m.nch1 : m.nch0;
            const int base = cls ? m.tap1 : m.tap0;
            for (int c = 0; c < nch; ++c)
                for (int lane = 0; lane < 64; ++lane)
                    for (int e = 0; e < 8; ++e)
                        tp[((size_t)(base + c) * 64 + lane) * 8 + e] =
                            host_bf16(tap_value(h, wd, delta, c, lane, e));
        }
    }
    // cost of one work item of row j (relative MFMA count)
    const int nlat_out = D.nlat_out;
    std::vector<double> cost(nlat_out, 0.0);
    for (int j = 0; j < nlat_out; ++j) {
        double c = 96.0;
        for (int64_t n = h.win_ptr[j]; n < h.win_ptr[j + 1]; ++n)
            c += 6.0 * (wins[n].nch0 + wins[n].nch1) + 8.0;
        cost[j] = c;
    }
    double total = 0.0;
    for (double c : cost) total += c;
    // contiguous bands of equal cost, one per XCD; heaviest rows first in a band
    std::vector<std::vector<int>> band(kNumXcd);
    {
        double acc = 0.0;
        for (int j = 0; j < nlat_out; ++j) {
            int k = (int)std::floor((acc + 0.5 * cost[j]) / total * kNumXcd);
            k = std::max(0, std::min(kNumXcd - 1, k));
            band[k].push_back(j);
            acc += cost[j];
        }
        for (auto& b : band)
            std::stable_sort(b.begin(), b.end(), [&](int a, int c) { return cost[a] > cost[c]; });
    }
    // info block
    info.assign(kInfoSize, 0);
    info[kInfoMagic] = 0x44495343;
    info[kInfoNwin] = nwin;
    info[kInfoWins] = (int32_t)info.size();
    const int* wp = reinterpret_cast<const int*>(wins.data());
    info.insert(info.end(), wp, wp + (size_t)nwin * (sizeof(MfmaWin) / 4));
    info[kInfoWinPtr] = (int32_t)info.size();
    for (int j = 0; j <= nlat_out; ++j) info.push_back((int32_t)h.win_ptr[j]);
    const int nqt = (D.nlon_out + kQ - 1) / kQ;
    size_t stride = 0;
    for (auto& bd : band) stride = std::max(stride, bd.size() * (size_t)nqt);
    const int base = (int)info.size();
    info[kInfoQ] = kQ;
    info[kInfoNqt] = nqt;
    info[kInfoWork] = base;
    info[kInfoStride] = (int32_t)stride;
    info.resize(info.size() + stride * kNumXcd, -1);
    for (int k = 0; k < kNumXcd; ++k) {
        size_t n = 0;
        for (int j : band[k])
            for (int qt = 0; qt < nqt; ++qt) info[base + k * stride + n++] = j * nqt + qt;
    }
    return DISCO_OK;
}

namespace {

__device__ __forceinline__ floatx16 mfma(const bf16x8_t& a, const bf16x8_t& b, const floatx16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Weights into operand fragments: frag f = ((chunk*16 + ks)*(Co/32) + mt)*64 + lane holds
// w[co = mt*32 + lane%32][ci = chunk*32 + 2*ks + lane/32][k = 0..7] (zero for k >= K).
__global__ __launch_bounds__(256) void prep_weight_frags(const bf16_t* __restrict__ w,
                                                          uint4* __restrict__ wf, int Ci, int Co,
                                                          int K) {
    const int f = blockIdx.x * 256 + threadIdx.x;
    const int nf = (Ci / 32) * 16 * (Co / 32) * 64;
    if (f >= nf) return;
    const int lane = f & 63;
    int r = f >> 6;
    const int mt = r % (Co / 32);
    r /= (Co / 32);
    const int ks = r % 16;
    const int chunk = r / 16;
    const int co = mt * 32 + (lane & 31);
    const int ci = chunk * 32 + 2 * ks + (lane >> 5);
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < K ? w[((size_t)co * Ci + ci) * K + e] : (uint16_t)0;
    uint4 o;
    o.x = v[0] | ((uint32_t)v[1] << 16);
    o.y = v[2] | ((uint32_t)v[3] << 16);
    o.z = v[4] | ((uint32_t)v[5] << 16);
    o.w = v[6] | ((uint32_t)v[7] << 16);
    wf[f] = o;
}

template <int S, int CO, int Q, int WM, int WN, typename TY>
__global__ __launch_bounds__(256, 1) void fused_mfma(
    const bf16_t* __restrict__ x, const uint4* __restrict__ wfrag, const float* __restrict__ bias,
    TY* __restrict__ y, const MfmaWin* __restrict__ wins, const int32_t* __restrict__ win_ptr,
    const uint4* __restrict__ taps, const int32_t* __restrict__ work, int work_stride, int nqt,
    int Ci, int nlat_in, int nlon_in, int nlat_out, int nlon_out) {
    constexpr int QW = Q / 4;            // outputs per wave in the contraction
    constexpr int NBW = QW / 4;          // 4-output blocks per wave
    constexpr int MT = CO / WM / 32;     // einsum M tiles per wave
    constexpr int NT = Q / WN / 32;      // einsum N tiles per wave
    constexpr int XKS = 256 + kXkPad;    // xk tile row stride (elements)
    static_assert(QW % 8 == 0, "wave output range must keep 8-alignment");

    __shared__ __attribute__((aligned(16))) bf16_t xk_lds[Q * XKS];
    __shared__ __attribute__((aligned(16))) bf16_t xs_lds[4 * 32 * kXsStride];

    const int xcd = blockIdx.x % kNumXcd;
    const int item = work[xcd * work_stride + blockIdx.x / kNumXcd];
    if (item < 0) return;
    const int b = blockIdx.y;
    const int j = item / nqt;
    const int q0 = (item % nqt) * Q;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lg = lane >> 5;           // lane group (k half of an operand)
    const int l32 = lane & 31;
    const int qwave = q0 + wave * QW;
    const int wm = wave / WN, wn = wave % WN;

    bf16_t* xs = xs_lds + wave * 32 * kXsStride;
    const size_t plane_in = (size_t)nlat_in * nlon_in;
    const int w_begin = win_ptr[j], w_end = win_ptr[j + 1];

    floatx16 g[MT][NT];
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) g[a][c][e] = 0.0f;

    const int nchunks = Ci / 32;
    for (int cc = 0; cc < nchunks; ++cc) {
        floatx16 acc[NBW];
#pragma unroll
        for (int n = 0; n < NBW; ++n)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[n][e] = 0.0f;
        const bf16_t* xc = x + ((size_t)b * Ci + (size_t)cc * 32) * plane_in;

        for (int wi = w_begin; wi < w_end; ++wi) {
            const MfmaWin m = wins[wi];
            const int d0 = m.p_lo & 7;
            const int nch = max(m.nch0, m.nch1);
            const int u0 = S * qwave + (m.p_lo & ~7);
            const bf16_t* xrow = xc + (size_t)m.lat * nlon_in;
            // fragment slot v(b) of 4-output block b: u_b = 8*floor((d0 + 4*S*b)/8)
            const bool hi = d0 >= 4;
            // chunks per staged piece
            const int vmax = (S == 1) ? (hi ? (NBW) / 2 : (NBW - 1) / 2) : (NBW - 1);
            const int cpp = 1 + (kXsLen - 16 - 8 * vmax) / 16;
            for (int c = 0; c < nch; c += cpp) {
                // ---- stage 32 channels x 128 longitudes starting at u0 + 16c ----
                lds_fence();
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int pr = lane + 64 * r;
                    const int ci = pr >> 4, grp = pr & 15;
                    const int gx = (u0 + 16 * c + 8 * grp) % nlon_in;
                    const uint4 v = *reinterpret_cast<const uint4*>(xrow + (size_t)ci * plane_in + gx);
                    *reinterpret_cast<uint4*>(xs + ci * kXsStride + 8 * grp) = v;
                }
                lds_fence();
                const int cend = min(nch, c + cpp);
                for (int k = c; k < cend; ++k) {
                    const int du = 16 * (k - c);
                    uint4 t0 = make_uint4(0, 0, 0, 0), t1 = make_uint4(0, 0, 0, 0);
                    if (k < m.nch0) t0 = taps[(size_t)(m.tap0 + k) * 64 + lane];
                    if ((S & 1) && k < m.nch1) t1 = taps[(size_t)(m.tap1 + k) * 64 + lane];
                    const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(&t0);
                    const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(&t1);
                    if (S == 1) {
                        constexpr int NV = NBW / 2 + 1;
                        bf16x8_t f[NV];
#pragma unroll
                        for (int v = 0; v < NV; ++v) {
                            const int u = du + 8 * v + 8 * lg;
                            f[v] = (u + 8 <= kXsLen)
                                       ? *reinterpret_cast<const bf16x8_t*>(xs + l32 * kXsStride + u)
                                       : f[0];
                        }
                        if (!hi) {
#pragma unroll
                            for (int n = 0; n < NBW; ++n) acc[n] = mfma((n & 1) ? a1 : a0, f[n / 2], acc[n]);
                        } else {
#pragma unroll
                            for (int n = 0; n < NBW; ++n)
                                acc[n] = mfma((n & 1) ? a1 : a0, f[(n + 1) / 2], acc[n]);
                        }
                    } else {
#pragma unroll
                        for (int n = 0; n < NBW; ++n) {
                            const int u = du + 8 * n + 8 * lg;
                            const bf16x8_t f = *reinterpret_cast<const bf16x8_t*>(xs + l32 * kXsStride + u);
                            acc[n] = mfma(a0, f, acc[n]);
                        }
                    }
                }
            }
        }
        // ---- xk tile: lane (ci = l32, lg) holds k = 4*lg + e%4 for qq = e/4 ----
        __syncthreads();   // previous chunk's GEMM finished reading xk_lds
#pragma unroll
        for (int n = 0; n < NBW; ++n) {
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int ql = wave * QW + 4 * n + qq;
                uint2 pk;
                pk.x = (uint32_t)f32_to_bf16(acc[n][4 * qq + 0]) |
                       ((uint32_t)f32_to_bf16(acc[n][4 * qq + 1]) << 16);
                pk.y = (uint32_t)f32_to_bf16(acc[n][4 * qq + 2]) |
                       ((uint32_t)f32_to_bf16(acc[n][4 * qq + 3]) << 16);
                *reinterpret_cast<uint2*>(xk_lds + ql * XKS + l32 * 8 + 4 * lg) = pk;
            }
        }
        __syncthreads();
        // ---- channel/basis GEMM over this chunk's 256 (ci, k) pairs ----
        const uint4* wf = wfrag + (size_t)cc * 16 * (CO / 32) * 64;
#pragma unroll 4
        for (int ks = 0; ks < 16; ++ks) {
            bf16x8_t af[MT], bf[NT];
#pragma unroll
            for (int a = 0; a < MT; ++a) {
                const uint4 v = wf[((size_t)ks * (CO / 32) + wm * MT + a) * 64 + lane];
                af[a] = *reinterpret_cast<const bf16x8_t*>(&v);
            }
#pragma unroll
            for (int c = 0; c < NT; ++c) {
                const int ql = wn * (Q / WN) + c * 32 + l32;
                bf[c] = *reinterpret_cast<const bf16x8_t*>(xk_lds + ql * XKS + ks * 16 + 8 * lg);
            }
#pragma unroll
            for (int a = 0; a < MT; ++a)
#pragma unroll
                for (int c = 0; c < NT; ++c) g[a][c] = mfma(af[a], bf[c], g[a][c]);
        }
    }
    // ---- epilogue ----
    TY* yb = y + (size_t)b * CO * nlat_out * nlon_out + (size_t)j * nlon_out;
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        const int q = q0 + wn * (Q / WN) + c * 32 + l32;
        if (q >= nlon_out) continue;
#pragma unroll
        for (int a = 0; a < MT; ++a) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int co = wm * (CO / WM) + a * 32 + 8 * (e >> 2) + 4 * lg + (e & 3);
                const float bv = bias ? bias[co] : 0.0f;
                store_f(yb, (size_t)co * nlat_out * nlon_out + q, g[a][c][e] + bv);
            }
        }
    }
}

}  // namespace

int try_launch_fused_mfma(const disco_psi* psi, const void* x, const void* w, const float* bias,
                          void* y, int y_dtype, int B, int Ci, int Co, int groups, hipStream_t st,
                          int* rc) {
    const DevPsi& d = psi->dev;
    const HostPsi& h = psi->host;
    if (!d.mfma_ok || groups != 1 || Ci % 32 != 0 || (Co != 128 && Co != 64) || h.K > 8) return 0;
    if ((reinterpret_cast<uintptr_t>(x) & 15) != 0) return 0;
    const int S = h.stride;
    if (S != 1 && S != 2) return 0;
    const int* hi = d.mfma_info_host.data();
    const int nqt = hi[kInfoNqt];
    const int woff = hi[kInfoWork];
    const int wstride = hi[kInfoStride];
    const int32_t* dinfo = d.mfma_row_info;
    const MfmaWin* wins = reinterpret_cast<const MfmaWin*>(dinfo + hi[kInfoWins]);
    const int32_t* win_ptr = dinfo + hi[kInfoWinPtr];
    const int32_t* work = dinfo + woff;
    const uint4* taps = static_cast<const uint4*>(d.mfma_taps);

    // weight fragments (stream-ordered workspace)
    const size_t nfrag = (size_t)(Ci / 32) * 16 * (Co / 32) * 64;
    void* wsp = nullptr;
    hipError_t e = hipMallocAsync(&wsp, nfrag * sizeof(uint4), st);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        *rc = set_error(e == hipErrorOutOfMemory ? DISCO_ENOMEM : DISCO_EHIP,
                        "hipMallocAsync for the weight fragments failed: %s", hipGetErrorString(e));
        return 1;
    }
    uint4* wf = static_cast<uint4*>(wsp);
    hipLaunchKernelGGL(prep_weight_frags, dim3((unsigned)((nfrag + 255) / 256)), dim3(256), 0, st,
                       static_cast<const bf16_t*>(w), wf, Ci, Co, h.K);
    const bf16_t* X = static_cast<const bf16_t*>(x);
    const disco_psi_desc& D = h.desc;
    dim3 grid((unsigned)(kNumXcd * wstride), (unsigned)B);
#define DISCO_FM(SS, CC, QQ, WMM, WNN, TT)                                                         \
    hipLaunchKernelGGL((fused_mfma<SS, CC, QQ, WMM, WNN, TT>), grid, dim3(256), 0, st, X, wf, bias, \
                       (TT*)y, wins, win_ptr, taps, work, wstride, nqt, Ci, D.nlat_in, D.nlon_in,   \
                       D.nlat_out, D.nlon_out)
    const bool f32 = y_dtype == DISCO_F32;
    if (Co == 128) {
        if (S == 1) { if (f32) DISCO_FM(1, 128, 128, 2, 2, float); else DISCO_FM(1, 128, 128, 2, 2, bf16_t); }
        else        { if (f32) DISCO_FM(2, 128, 128, 2, 2, float); else DISCO_FM(2, 128, 128, 2, 2, bf16_t); }
    } else {
        if (S == 1) { if (f32) DISCO_FM(1, 64, 128, 2, 2, float); else DISCO_FM(1, 64, 128, 2, 2, bf16_t); }
        else        { if (f32) DISCO_FM(2, 64, 128, 2, 2, float); else DISCO_FM(2, 64, 128, 2, 2, bf16_t); }
    }
#undef DISCO_FM
    hipError_t le = hipGetLastError();
    hipError_t fe = hipFreeAsync(wsp, st);
    if (le != hipSuccess) {
        *rc = set_error(DISCO_EHIP, "fused_mfma launch failed: %s", hipGetErrorString(le));
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
