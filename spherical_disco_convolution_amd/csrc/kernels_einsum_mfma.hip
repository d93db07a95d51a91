// Channel/basis contraction of the DISCO forward pass on CDNA4 matrix cores.
//
//   y[b, co, n] = bias[co] + sum_{kappa} w[co, kappa] * xk[b, G(co)*Ci/G*K + kappa, n]
//
// kappa = ci'*K + k runs over the group's (channel, basis) pairs; with the
// [B, Ci, K, H, W] layout of xk these rows are contiguous, so per (batch,
// group) this is a dense GEMM  C[cog x HW] = A[cog x Kd] * B[Kd x HW]  with
// Kd = (Ci/G)*K (DiscreteContinuousConvS2 page, forward equation: the sums
// over c_i and k).  bf16 operands, float32 accumulation with
// v_mfma_f32_32x32x16_bf16.
//
// General tiling (any group size): a 256-thread workgroup computes a BM x 128
// tile of C and walks Kd in steps of 32.  A (weights) is staged as [m][k]; B (xk) is staged transposed,
// [n][k], so that each lane's eight consecutive k values are one 16-byte LDS
// read, the operand layout the MFMA wants.  Rows are padded by 8 elements so
// the 16-byte reads of 16 consecutive rows hit distinct banks.
#include <hip/hip_runtime.h>

#include "disco_internal.h"
#include "kernels_common.h"

namespace disco {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int BN = 128;
constexpr int BK = 32;
constexpr int LDK = BK + 8;   // padded row length (elements)

template <int BM, typename TY>
__global__ __launch_bounds__(256) void einsum_mfma_bf16(const bf16_t* __restrict__ xk,
                                                        const bf16_t* __restrict__ w,
                                                        const float* __restrict__ bias,
                                                        TY* __restrict__ y, int Ci, int Co,
                                                        int groups, int K, int HW, int vec_ok) {
    __shared__ __attribute__((aligned(16))) bf16_t As[BM * LDK];
    __shared__ __attribute__((aligned(16))) bf16_t Bs[BN * LDK];

    const int n0 = blockIdx.x * BN;
    const int m0 = blockIdx.y * BM;          // within the group
    const int bg = blockIdx.z;
    const int b = bg / groups, grp = bg % groups;
    const int cig = Ci / groups, cog = Co / groups;
    const int Kd = cig * K;
    const bf16_t* A = w + (size_t)grp * cog * Kd;
    const bf16_t* Bm = xk + ((size_t)b * Ci + (size_t)grp * cig) * K * (size_t)HW;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // wave tiling: BM = 128 -> 2 x 2 waves of 64 x 64; BM = 64 -> 1 x 4 waves of 64 x 32
    constexpr int WN = (BM == 128) ? 64 : 32;
    constexpr int NT = WN / 32;               // 32-wide MFMA tiles per wave along n
    const int wm = (BM == 128) ? (wave >> 1) : 0;
    const int wn = (BM == 128) ? (wave & 1) : wave;

    floatx16 acc[2][NT];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][c][e] = 0.0f;

    for (int k0 = 0; k0 < Kd; k0 += BK) {
        // ---- stage A: BM x 32, thread -> (row, 16 consecutive k) ----
        for (int idx = tid; idx < BM * 2; idx += 256) {
            const int m = idx >> 1, kh = (idx & 1) * 16;
            const int gm = m0 + m, gk = k0 + kh;
            u16x8 v0, v1;
            if (gm < cog && vec_ok && gk + 16 <= Kd) {
                const u16x8* src = reinterpret_cast<const u16x8*>(A + (size_t)gm * Kd + gk);
                v0 = src[0];
                v1 = src[1];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    v0[e] = (gm < cog && gk + e < Kd) ? A[(size_t)gm * Kd + gk + e] : 0;
                    v1[e] = (gm < cog && gk + 8 + e < Kd) ? A[(size_t)gm * Kd + gk + 8 + e] : 0;
                }
            }
            *reinterpret_cast<u16x8*>(&As[m * LDK + kh]) = v0;
            *reinterpret_cast<u16x8*>(&As[m * LDK + kh + 8]) = v1;
        }
        // ---- stage B transposed: thread -> (n pair, 8 consecutive k) ----
        {
            const int np = tid & 63, kg = tid >> 6;
            const int gn = n0 + 2 * np;
            u16x8 c0, c1;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int gk = k0 + kg * 8 + e;
                uint16_t a0 = 0, a1 = 0;
                if (gk < Kd) {
                    const bf16_t* row = Bm + (size_t)gk * HW;
                    if (vec_ok && gn + 1 < HW) {
                        const uint32_t pr = *reinterpret_cast<const uint32_t*>(row + gn);
                        a0 = (uint16_t)(pr & 0xffffu);
                        a1 = (uint16_t)(pr >> 16);
                    } else {
                        if (gn < HW) a0 = row[gn];
                        if (gn + 1 < HW) a1 = row[gn + 1];
                    }
                }
                c0[e] = a0;
                c1[e] = a1;
            }
            *reinterpret_cast<u16x8*>(&Bs[(2 * np) * LDK + kg * 8]) = c0;
            *reinterpret_cast<u16x8*>(&Bs[(2 * np + 1) * LDK + kg * 8]) = c1;
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < BK; ks += 16) {
            bf16x8_t af[2], bfr[NT];
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                const int m = wm * 64 + a * 32 + (lane & 31);
                af[a] = *reinterpret_cast<const bf16x8_t*>(&As[m * LDK + ks + 8 * (lane >> 5)]);
            }
#pragma unroll
            for (int c = 0; c < NT; ++c) {
                const int n = wn * WN + c * 32 + (lane & 31);
                bfr[c] = *reinterpret_cast<const bf16x8_t*>(&Bs[n * LDK + ks + 8 * (lane >> 5)]);
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int c = 0; c < NT; ++c)
                    acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[c], acc[a][c],
                                                                       0, 0, 0);
        }
        __syncthreads();
    }
    // ---- epilogue: lane holds column n = lane%32, rows 8*(e/4) + 4*(lane/32) + e%4 ----
    TY* Y = y + ((size_t)b * Co + (size_t)grp * cog) * HW;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int c = 0; c < NT; ++c) {
            const int n = n0 + wn * WN + c * 32 + (lane & 31);
            if (n >= HW) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + wm * 64 + a * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (m < cog) {
                    const float bv = bias ? bias[grp * cog + m] : 0.0f;
                    store_f(Y, (size_t)m * HW + n, acc[a][c][e] + bv);
                }
            }
        }
    }
}

// --------------------------------------------------------------------------
// Streamed variant for a group of 64 or 128 output channels and Kd % 32 == 0
// (the shapes of a layer's channel/basis contraction): one 512-thread
// workgroup computes all cog rows for 256 output points, walking Kd in steps
// of 32 with the next step's global loads in flight while the matrix cores
// work on the current one, and one barrier per step (double-buffered LDS).
//
// xk is staged transposed, [n][kappa], so that the B operand is one 16-byte
// LDS read per lane.  A thread loads 16 bytes (8 points) of two consecutive
// kappa rows and writes 8 kappa pairs; a wave's loads cover 128-byte row
// segments.  The 16-byte kappa chunks of row n sit at chunk ^ ((n >> 3) & 3),
// which spreads the pair writes of eight point-octets over the banks.
// --------------------------------------------------------------------------
constexpr int SN = 256;         // output points per workgroup
constexpr int SK = 32;          // kappa per step
constexpr int SLD = SK + 8;     // LDS row (elements): 80 bytes, 16-byte aligned

template <int BM, typename TY>
__global__ __launch_bounds__(512) void einsum_stream_bf16(const bf16_t* __restrict__ xk,
                                                          const bf16_t* __restrict__ w,
                                                          const float* __restrict__ bias,
                                                          TY* __restrict__ y, int Ci, int Co,
                                                          int groups, int K, int HW) {
    __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * SLD];
    __shared__ __attribute__((aligned(16))) bf16_t Bs[2][SN * SLD];
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

    const int n0 = blockIdx.x * SN;
    const int bg = blockIdx.y;
    const int b = bg / groups, grp = bg % groups;
    const int cig = Ci / groups;
    const int Kd = cig * K;
    const bf16_t* A = w + (size_t)grp * BM * Kd;
    const bf16_t* Bm = xk + ((size_t)b * Ci + (size_t)grp * cig) * K * (size_t)HW;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int l32 = lane & 31, lg = lane >> 5;
    // wave grid: BM = 128 -> 2 x 4 waves of 64 x 64; BM = 64 -> 1 x 8 waves of 64 x 32
    constexpr int WNW = BM == 128 ? 4 : 8;
    constexpr int WTN = SN / WNW;
    constexpr int NT = WTN / 32;
    const int wm = wave / WNW, wn = wave % WNW;

    // B load task: kappa pair kp (rows 2kp, 2kp+1 of the step), point octet oc
    const int kp = (lane & 7) + 8 * (wave & 1);
    const int oc = (lane >> 3) + 8 * (wave >> 1);
    const int gn = n0 + 8 * oc;
    const bool bvalid = gn < HW;   // HW % 8 == 0: an octet is wholly in or out
    const bf16_t* bsrc = Bm + (size_t)(2 * kp) * HW + (bvalid ? gn : 0);
    const int bdst = (8 * oc) * SLD + 8 * ((kp >> 2) ^ (oc & 3)) + 2 * (kp & 3);
    // A load task: row am, 8 kappa at 8 * ac
    const int am = tid >> 2, ac = tid & 3;
    const bool aload = am < BM;
    const bf16_t* asrc = A + (size_t)(aload ? am : 0) * Kd + 8 * ac;
    const int adst = am * SLD + 8 * ac;

    u32x4v pa = {0, 0, 0, 0}, pb0 = {0, 0, 0, 0}, pb1 = {0, 0, 0, 0};
    auto gload = [&](int k0) {
        if (aload) pa = *reinterpret_cast<const u32x4v*>(asrc + k0);
        if (bvalid) {
            pb0 = *reinterpret_cast<const u32x4v*>(bsrc + (size_t)k0 * HW);
            pb1 = *reinterpret_cast<const u32x4v*>(bsrc + (size_t)(k0 + 1) * HW);
        }
    };
    auto lstore = [&](int buf) {
        if (aload) *reinterpret_cast<u32x4v*>(&As[buf][adst]) = pa;
        bf16_t* bd = &Bs[buf][bdst];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t lo = pb0[i >> 1], hi = pb1[i >> 1];
            const uint32_t wd = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                        : ((lo & 0xffffu) | (hi << 16));
            *reinterpret_cast<uint32_t*>(bd + i * SLD) = wd;
        }
    };

    // per-lane LDS offsets of the operands (elements)
    int aoff[2], boff[NT][2];
#pragma unroll
    for (int a = 0; a < 2; ++a) aoff[a] = (wm * 64 + a * 32 + l32) * SLD + 8 * lg;
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        const int n = wn * WTN + c * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) boff[c][ks] = n * SLD + 8 * ((2 * ks + lg) ^ ((n >> 3) & 3));
    }

    floatx16 acc[2][NT];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][c][e] = 0.0f;

    gload(0);
    lstore(0);
    __syncthreads();
    int buf = 0;
    for (int k0 = 0; k0 < Kd; k0 += SK) {
        const bool more = k0 + SK < Kd;
        if (more) gload(k0 + SK);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8_t af[2], bfr[NT];
#pragma unroll
            for (int a = 0; a < 2; ++a)
                af[a] = *reinterpret_cast<const bf16x8_t*>(&As[buf][aoff[a] + 16 * ks]);
#pragma unroll
            for (int c = 0; c < NT; ++c)
                bfr[c] = *reinterpret_cast<const bf16x8_t*>(&Bs[buf][boff[c][ks]]);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int c = 0; c < NT; ++c)
                    acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[c], acc[a][c],
                                                                       0, 0, 0);
        }
        if (more) lstore(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }
    // ---- epilogue: lane holds point n = lane % 32, rows 8*(e/4) + 4*(lane/32) + e%4 ----
    TY* Y = y + ((size_t)b * Co + (size_t)grp * BM) * HW;
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        const int n = n0 + wn * WTN + c * 32 + l32;
        if (n >= HW) continue;
#pragma unroll
        for (int a = 0; a < 2; ++a) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = wm * 64 + a * 32 + 8 * (e >> 2) + 4 * lg + (e & 3);
                const float bv = bias ? bias[grp * BM + m] : 0.0f;
                store_f(Y, (size_t)m * HW + n, acc[a][c][e] + bv);
            }
        }
    }
}

}  // namespace

int launch_einsum_mfma_bf16(const void* xk, const void* w, const float* bias, void* y, int y_dtype,
                            int B, int Ci, int Co, int groups, int K, int HW, hipStream_t st) {
    const int cog = Co / groups, cig = Ci / groups;
    const int Kd = cig * K;
    const int vec_ok = (Kd % 8 == 0) && (HW % 2 == 0) &&
                       ((reinterpret_cast<uintptr_t>(w) & 15) == 0) &&
                       ((reinterpret_cast<uintptr_t>(xk) & 3) == 0);
    const bf16_t* X = static_cast<const bf16_t*>(xk);
    const bf16_t* Wt = static_cast<const bf16_t*>(w);
    if ((cog == 128 || cog == 64) && Kd % SK == 0 && HW % 8 == 0 &&
        (reinterpret_cast<uintptr_t>(w) & 15) == 0 && (reinterpret_cast<uintptr_t>(xk) & 15) == 0) {
        dim3 sgrid((HW + SN - 1) / SN, B * groups);
#define DISCO_ES(BMV, TT)                                                                        \
    hipLaunchKernelGGL((einsum_stream_bf16<BMV, TT>), sgrid, dim3(512), 0, st, X, Wt, bias, (TT*)y, \
                       Ci, Co, groups, K, HW)
        {
            KernelTimer timer("einsum_stream_bf16", st);
            if (cog == 128) {
                if (y_dtype == DISCO_F32) DISCO_ES(128, float);
                else DISCO_ES(128, bf16_t);
            } else {
                if (y_dtype == DISCO_F32) DISCO_ES(64, float);
                else DISCO_ES(64, bf16_t);
            }
        }
#undef DISCO_ES
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return set_error(DISCO_EHIP, "einsum_stream launch failed: %s", hipGetErrorString(e));
        return DISCO_OK;
    }
    const int BM = cog > 64 ? 128 : 64;
    dim3 grid((HW + BN - 1) / BN, (cog + BM - 1) / BM, B * groups);
    KernelTimer timer("einsum_mfma_bf16", st);
    if (BM == 128) {
        if (y_dtype == DISCO_F32)
            hipLaunchKernelGGL((einsum_mfma_bf16<128, float>), grid, dim3(256), 0, st, X, Wt, bias,
                               (float*)y, Ci, Co, groups, K, HW, vec_ok);
        else
            hipLaunchKernelGGL((einsum_mfma_bf16<128, bf16_t>), grid, dim3(256), 0, st, X, Wt, bias,
                               (bf16_t*)y, Ci, Co, groups, K, HW, vec_ok);
    } else {
        if (y_dtype == DISCO_F32)
            hipLaunchKernelGGL((einsum_mfma_bf16<64, float>), grid, dim3(256), 0, st, X, Wt, bias,
                               (float*)y, Ci, Co, groups, K, HW, vec_ok);
        else
            hipLaunchKernelGGL((einsum_mfma_bf16<64, bf16_t>), grid, dim3(256), 0, st, X, Wt, bias,
                               (bf16_t*)y, Ci, Co, groups, K, HW, vec_ok);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return set_error(DISCO_EHIP, "einsum_mfma launch failed: %s", hipGetErrorString(e));
    return DISCO_OK;
}

}  // namespace disco
