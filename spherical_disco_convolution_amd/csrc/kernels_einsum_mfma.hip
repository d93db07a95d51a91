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

#include <algorithm>
#include <cstdlib>
#include <cstring>

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

// --------------------------------------------------------------------------
// Ring-pipelined variant for one channel group of 64 or 128 output channels
// (Kd % 32 == 0, HW % 8 == 0, HW >= 256): one workgroup per CU walks its
// output tiles (256 points by every output channel) as a single stream of
// 32-kappa steps.  Two copy waves move each step's operands -- the weights
// [BM][32] and the X_K block [32 kappa][256 points] -- from global memory
// straight into a ring of NS LDS stages (global_load_lds), NS - 1 steps ahead
// of the eight matrix-core waves and across tile boundaries; one barrier per
// step hands a stage over.  Only the copy waves wait on vector-memory counts,
// and they issue nothing else, so every wait is exact; the matrix-core waves
// only read LDS and store results.
//
// The X_K block stays as it is in memory, points contiguous, its 16-byte
// chunks permuted within a row by chunk ^ 4 (kappa & 3); ds_read_b64_tr_b16
// then hands each lane four kappa of one point, two such reads one operand
// fragment.  The weight rows (64 bytes) hold their chunks at chunk ^ ((row >> 2) & 3).
// Both permutations make the operand reads of a half-wave cover all LDS banks.
//
// The last tile of a row of points is shifted back to end at HW, so every
// tile is whole; its leading points repeat columns of the tile before, and
// both write the same values.
// --------------------------------------------------------------------------
constexpr int RN = 256;                    // output points per tile
constexpr int RK = 32;                     // kappa per step
constexpr int RB_BYTES = RK * RN * 2;      // X_K block of a stage: 16 KiB
constexpr int R_COPY_WAVES = 2;
constexpr int R_MMA_WAVES = 8;
constexpr int R_THREADS = 64 * (R_COPY_WAVES + R_MMA_WAVES);

template <int BM>
struct RingCfg {
    static constexpr int A_BYTES = BM * RK * 2;           // weight slice: 8 / 4 KiB
    static constexpr int STAGE = A_BYTES + RB_BYTES;      // 24 / 20 KiB
    static constexpr int NS = BM == 128 ? 6 : 7;          // 144 / 140 KiB of LDS
    static constexpr int A_INS = A_BYTES / 1024;          // copy instructions per step
    static constexpr int B_INS = RB_BYTES / 1024;
    static constexpr int OPS = (A_INS + B_INS) / R_COPY_WAVES;   // per copy wave
    static constexpr int WNW = BM == 128 ? 4 : 8;         // matrix-core waves along the points
    static constexpr int WTN = RN / WNW;                  // 64 / 32 points per wave
    static constexpr int NT = WTN / 32;
    static_assert((A_INS + B_INS) % R_COPY_WAVES == 0, "copy split");
    static_assert(OPS * (NS - 2) < 64, "vmcnt range");
};

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ void store_nt(float* p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_nt(bf16_t* p, float v) {
    __builtin_nontemporal_store(f32_to_bf16(v), p);
}

template <int BM, typename TY>
__global__ __launch_bounds__(R_THREADS) void einsum_ring_bf16(const bf16_t* __restrict__ xk,
                                                              const bf16_t* __restrict__ w,
                                                              const float* __restrict__ bias,
                                                              TY* __restrict__ y, int Kd, int HW,
                                                              int ntiles) {
    using C = RingCfg<BM>;
    constexpr int NS = C::NS;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[NS * C::STAGE];
    __shared__ __attribute__((aligned(16))) float bias_s[BM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int nk = Kd / RK;
    const int ntn = (HW + RN - 1) / RN;
    const int G = gridDim.x;
    // Tiles base, base + G, ...  Workgroups go to the 8 XCDs round-robin; base
    // gives the G / 8 workgroups of one XCD consecutive tiles, so that the
    // cache lines two neighbouring tiles share (X_K rows need not start on a
    // line) are fetched once into that XCD's L2.
    const int bx = (int)blockIdx.x;
    const int base = G % 8 == 0 ? (bx % 8) * (G / 8) + bx / 8 : bx;
    const int my_tiles = base < ntiles ? (ntiles - 1 - base) / G + 1 : 0;
    const int Q = my_tiles * nk;   // steps of this workgroup
    if (Q == 0) return;

    if (wave >= R_MMA_WAVES) {
        // ---------------- copy waves ----------------
        const int cw = wave - R_MMA_WAVES;
        const uint32_t ring_lds =
            __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void*)&ring[0]);
        // the wave takes copy instructions cw, cw + 2, ...: its first A_INS / 2
        // move weight rows 16 i .. 16 i + 15, the rest X_K rows 2 j, 2 j + 1
        // (j = i - A_INS).  This lane's source offsets (elements) and LDS
        // offsets of each:
        constexpr int OA = C::A_INS / R_COPY_WAVES;
        int64_t src_off[C::OPS];
        uint32_t dst_off[C::OPS];
#pragma unroll
        for (int o = 0; o < C::OPS; ++o) {
            const int i = cw + R_COPY_WAVES * o;
            if (o < OA) {
                const int P = 64 * i + lane;   // 16-byte slot of the weight slice
                const int row = P >> 2, c = (P & 3) ^ ((row >> 2) & 3);
                src_off[o] = (int64_t)row * Kd + 8 * c;
                dst_off[o] = (uint32_t)(1024 * i);
            } else {
                const int P = 64 * (i - C::A_INS) + lane;   // 16-byte slot of the X_K block
                const int kap = P >> 5, c = (P & 31) ^ (4 * (kap & 3));
                src_off[o] = (int64_t)kap * HW + 8 * c;
                dst_off[o] = (uint32_t)(C::A_BYTES + 1024 * (i - C::A_INS));
            }
        }
        // issue cursor: step ik of tile ti, ring stage iq
        int ik = 0, ti = base, iq = 0;
        int64_t xbase = 0;
        auto tile_base = [&]() {
            const int bb = ti / ntn, n0 = min((ti % ntn) * RN, HW - RN);
            xbase = (int64_t)bb * Kd * HW + n0;
        };
        tile_base();
        auto issue = [&]() {
            const uint32_t st = ring_lds + (uint32_t)(iq * C::STAGE);
            // past the last step every lane reloads 16 bytes of the weights
            // (cached), so that every step issues the same number of operations
            const bool live = ti < ntiles;
            const bf16_t* pa = live ? w + (int64_t)ik * RK : w;
            const bf16_t* pb = live ? xk + xbase + (int64_t)ik * RK * HW : w;
#pragma unroll
            for (int o = 0; o < C::OPS; ++o) {
                const int64_t off = live ? src_off[o] : (int64_t)lane * 8;
                dma_lds16((o < OA ? pa : pb) + off, st + dst_off[o]);
            }
            if (++iq == NS) iq = 0;
            if (++ik == nk) {
                ik = 0;
                ti += G;
                if (ti < ntiles) tile_base();
            }
        };
#pragma unroll 1
        for (int q = 0; q < NS - 1; ++q) issue();
#pragma unroll 1
        for (int q = 0; q < Q; ++q) {
            wait_vmcnt<C::OPS*(NS - 2)>();   // this wave's part of step q has landed
            __syncthreads();
            issue();                         // step q + NS - 1, into the stage read at step q - 1
        }
        wait_vmcnt<0>();   // no copy may land after the workgroup ends
        return;
    }

    // ---------------- matrix-core waves ----------------
    const int l32 = lane & 31, lg = lane >> 5;
    const int wm = wave / C::WNW, wn = wave % C::WNW;
    // weight fragment (second operand): row m, kappa 8 lg + 16 ks .. + 7
    uint32_t aoff[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int m = wm * 64 + l32;
        aoff[ks] = (uint32_t)(m * 64 + 16 * ((2 * ks + lg) ^ ((l32 >> 2) & 3)));
    }
    // X_K fragment (first operand) by two transposed reads: within each
    // 16-lane group, lane s reads kappa row 8 lg + 4 h + s / 4, points
    // 16 (group & 1) + 4 (s & 3) .. + 3 of the 32-point tile
    uint32_t boff[C::NT];
    {
        const int s = lane & 15, g = lane >> 4;
        const int kap = 8 * (g >> 1) + (s >> 2);
#pragma unroll
        for (int c = 0; c < C::NT; ++c) {
            const int n = wn * C::WTN + 32 * c + 16 * (g & 1) + 4 * (s & 3);
            boff[c] = (uint32_t)(C::A_BYTES + kap * 512 + 16 * ((n >> 3) ^ (4 * (kap & 3))) +
                                 2 * (n & 7));
        }
    }
    // bias rows in LDS (visible after the first step's barrier)
    for (int m = tid; m < BM; m += 64 * R_MMA_WAVES) bias_s[m] = bias ? bias[m] : 0.0f;

    floatx16 acc[2][C::NT];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < C::NT; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][c][e] = 0.0f;

    const lds_u8* ring_p = (const lds_u8*)&ring[0];
    int ck = 0, ti = base;
#pragma unroll 1
    for (int q = 0; q < Q; ++q) {
        __syncthreads();
        const lds_u8* st = ring_p + (q % NS) * C::STAGE;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8_t af[2], bfr[C::NT];
#pragma unroll
            for (int a = 0; a < 2; ++a)
                af[a] = *(const lds_bf16x8*)(st + aoff[ks] + a * 32 * 64);
#pragma unroll
            for (int c = 0; c < C::NT; ++c) {
                const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4i16*)(st + boff[c] + (16 * ks) * 512));
                const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4i16*)(st + boff[c] + (16 * ks + 4) * 512));
                const auto v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                bfr[c] = __builtin_bit_cast(bf16x8_t, v);
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int c = 0; c < C::NT; ++c)
                    acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[c], acc[a][c],
                                                                       0, 0, 0);
        }
        if (++ck == nk) {
            // lane holds point lane % 32 and rows 8 (e / 4) + 4 (lane / 32) + e % 4
            // of each 32 x 32 tile: a store instruction writes two whole
            // 128-byte row segments.  Streaming (non-temporal) stores keep the
            // results from displacing cached operands.
            const int bb = ti / ntn, n0 = min((ti % ntn) * RN, HW - RN);
            TY* Y = y + (size_t)bb * BM * HW;
#pragma unroll
            for (int a = 0; a < 2; ++a) {
#pragma unroll
                for (int eq = 0; eq < 4; ++eq) {
                    const int m0 = wm * 64 + 32 * a + 8 * eq + 4 * lg;
                    const float4 bq = *reinterpret_cast<const float4*>(&bias_s[m0]);
#pragma unroll
                    for (int c = 0; c < C::NT; ++c) {
                        const int n = n0 + wn * C::WTN + 32 * c + l32;
                        TY* p = Y + (size_t)m0 * HW + n;
                        store_nt(p, acc[a][c][4 * eq] + bq.x);
                        store_nt(p + HW, acc[a][c][4 * eq + 1] + bq.y);
                        store_nt(p + 2 * (size_t)HW, acc[a][c][4 * eq + 2] + bq.z);
                        store_nt(p + 3 * (size_t)HW, acc[a][c][4 * eq + 3] + bq.w);
                    }
                }
#pragma unroll
                for (int c = 0; c < C::NT; ++c)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[a][c][e] = 0.0f;
            }
            ck = 0;
            ti += G;
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
    // DISCO_EINSUM_PATH=stream selects the double-buffered kernel below
    const char* ev = std::getenv("DISCO_EINSUM_PATH");
    const bool ring_ok = !(ev && std::strcmp(ev, "stream") == 0);
    const int ring_ns = cog == 128 ? RingCfg<128>::NS : RingCfg<64>::NS;
    if (ring_ok && groups == 1 && (cog == 128 || cog == 64) && Kd % RK == 0 &&
        Kd / RK >= ring_ns - 1 && HW % 8 == 0 && HW >= RN &&
        (reinterpret_cast<uintptr_t>(w) & 15) == 0 && (reinterpret_cast<uintptr_t>(xk) & 15) == 0 &&
        (reinterpret_cast<uintptr_t>(y) & 15) == 0) {
        int dev = 0, ncu = 256;
        if (hipGetDevice(&dev) == hipSuccess)
            (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        const int ntiles = B * ((HW + RN - 1) / RN);
        const int grid = std::max(1, std::min(ntiles, ncu));   // one workgroup per CU (LDS)
#define DISCO_ER(BMV, TT)                                                                         \
    hipLaunchKernelGGL((einsum_ring_bf16<BMV, TT>), dim3(grid), dim3(R_THREADS), 0, st, X, Wt, bias, \
                       (TT*)y, Kd, HW, ntiles)
        {
            KernelTimer timer("einsum_ring_bf16", st);
            if (cog == 128) {
                if (y_dtype == DISCO_F32) DISCO_ER(128, float);
                else DISCO_ER(128, bf16_t);
            } else {
                if (y_dtype == DISCO_F32) DISCO_ER(64, float);
                else DISCO_ER(64, bf16_t);
            }
        }
#undef DISCO_ER
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return set_error(DISCO_EHIP, "einsum_ring launch failed: %s", hipGetErrorString(e));
        return DISCO_OK;
    }
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
