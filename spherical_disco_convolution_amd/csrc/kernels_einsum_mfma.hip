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
// Tiling: a 256-thread workgroup computes a BM x 128 tile of C and walks Kd in
// steps of 32.  A (weights) is staged as [m][k]; B (xk) is staged transposed,
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

}  // namespace

int launch_einsum_mfma_bf16(const void* xk, const void* w, const float* bias, void* y, int y_dtype,
                            int B, int Ci, int Co, int groups, int K, int HW, hipStream_t st) {
    const int cog = Co / groups, cig = Ci / groups;
    const int Kd = cig * K;
    const int vec_ok = (Kd % 8 == 0) && (HW % 2 == 0) &&
                       ((reinterpret_cast<uintptr_t>(w) & 15) == 0) &&
                       ((reinterpret_cast<uintptr_t>(xk) & 3) == 0);
    const int BM = cog > 64 ? 128 : 64;
    dim3 grid((HW + BN - 1) / BN, (cog + BM - 1) / BM, B * groups);
    const bf16_t* X = static_cast<const bf16_t*>(xk);
    const bf16_t* Wt = static_cast<const bf16_t*>(w);
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
