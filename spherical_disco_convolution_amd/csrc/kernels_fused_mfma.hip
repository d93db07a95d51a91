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
// One workgroup (4 waves) owns one output row and Q = 128 output longitudes
// for all output channels; each wave contracts 32 of the longitudes.  The
// input is walked in "pieces" (one window, up to 6 chunks of 16 longitudes,
// 32 channels); a piece's input and its first tap fragments are loaded into
// registers one piece ahead, so their latency overlaps the previous piece's
// matrix work.  Work items are spread over the 8 XCDs in contiguous latitude
// bands of equal cost (the polar rows carry ~100x more taps than the
// equatorial ones), so that workgroups sharing input rows share an L2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

#include "disco_internal.h"
#include "kernels_common.h"

namespace disco {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // 8 bf16 as a native vector
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));   // converts with v_cvt_pk_bf16_f32 (RNE)

constexpr int kNumXcd = 8;
constexpr int kQ = 128;             // output longitudes per work item
constexpr int kNbw = kQ / 16;       // 4-output blocks per wave
constexpr int kRing = 4;            // LDS ring slots: three pieces in flight while one is consumed
constexpr int kXkStride = 264;      // xk tile row: 256 (ci, k) pairs + 8 pad
constexpr int kXkTStride = 136;     // transposed xk tile row (k, ci): 128 outputs + 8 pad
constexpr int kGemmSteps = 4;       // GEMM k-steps (16 kappa each) per streamed weight piece
// Chunks of 16 input longitudes per contraction piece.
constexpr int cp_max(int S) { return S == 1 ? 4 : 2; }
// 16-byte groups per channel row that a piece of `cp` chunks reads: the last
// wave's last block reaches longitude S*96 + 8*floor((7 + 4*S*7)/8) + 16*(cp-1) + 15.
constexpr int piece_groups(int S, int cp) { return S == 1 ? 16 + 2 * cp : 31 + 2 * cp; }
// Staged row stride in 16-byte groups (odd: the 32 channel rows fall in distinct banks).
constexpr int row_stride(int S) { return piece_groups(S, cp_max(S)) | 1; }
constexpr int x_instr(int S) { return (32 * row_stride(S) + 63) / 64; }   // DMA loads of one strip
constexpr int tap_instr(int S) { return S == 1 ? 2 * cp_max(1) : cp_max(2); }
constexpr int slot_size(int S) { return (x_instr(S) + tap_instr(S)) * 64; }   // 16-byte units

struct MfmaWin {
    int32_t lat, p_lo, width, nch0, nch1, tap0, tap1, pad;
};

// One contraction piece: a window's input strip (up to cp_max chunks of 16
// longitudes) and its tap fragments.  32 bytes, read with scalar loads.
struct PieceDesc {
    int32_t xoff;    // input row offset within a channel plane (lat * nlon_in)
    int32_t uoff;    // first staged longitude before the work item's shift, in [0, nlon_in)
    int32_t tap0;    // tap fragment of chunk 0 of this piece, alignment class 0
    int32_t tap1;    // same for class 1 (odd strides)
    int32_t nck;     // chunks in this piece
    int32_t d0;      // window start modulo 8
    int32_t nv0;     // chunks with class-0 taps (the rest are zero)
    int32_t nv1;     // chunks with class-1 taps
};
static_assert(sizeof(PieceDesc) == 32, "descriptor layout");

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

// Layout of `info` (int32): header, piece_ptr[nlat_out+1], the PieceDesc array
// (8 ints each, 8-aligned), and the work items (j, q0, first piece, piece
// count) of all XCDs, each XCD's list contiguous and in (row, longitude tile)
// order.
enum { kInfoMagic = 0, kInfoPiecePtr, kInfoPieces, kInfoItems, kInfoNpieces, kInfoXcdOff,
       kInfoXcdLen = kInfoXcdOff + kNumXcd, kInfoSize = kInfoXcdLen + kNumXcd };

int build_mfma_tables(disco_psi* psi, std::vector<char>& taps, std::vector<int32_t>& info) {
    taps.clear();
    info.clear();
    const HostPsi& h = psi->host;
    const disco_psi_desc& D = h.desc;
    // The matrix-core path covers K <= 8, longitudes a multiple of 8 and
    // strides 1 and 2 (the latter: one alignment class).
    if (h.K > 8 || D.nlon_in % 8 != 0 || h.stride > 2 || D.nlon_in > 65536) return DISCO_OK;
    const int S = h.stride;
    const int cp = cp_max(S);
    const int nwin = (int)h.windows.size();
    const int nlat_out = D.nlat_out;
    std::vector<MfmaWin> wins(nwin);
    // fragment 0 is all zero: chunks beyond a class's band load it
    size_t nfrag = 1;
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
    // pieces: a window's chunks in groups of at most cp; an output row without
    // support gets one piece with zero taps so that its tile is still written
    std::vector<int32_t> piece_ptr(nlat_out + 1, 0);
    std::vector<PieceDesc> pieces;
    std::vector<double> cost(nlat_out, 0.0);
    for (int j = 0; j < nlat_out; ++j) {
        // relative cost of one work item of this row: a fixed part (weight
        // pieces, epilogue) plus per contraction piece and per chunk; the
        // weights are a least-squares fit of measured item times at 721x1440
        double c = 17.17;
        for (int64_t n = h.win_ptr[j]; n < h.win_ptr[j + 1]; ++n) {
            const MfmaWin& m = wins[n];
            const int nch = std::max(m.nch0, m.nch1);
            for (int c0 = 0; c0 < nch; c0 += cp) {
                PieceDesc pd;
                pd.xoff = m.lat * D.nlon_in;
                pd.uoff = (int32_t)(((int64_t)(m.p_lo & ~7) + 16 * c0) % D.nlon_in);
                pd.nck = std::min(cp, nch - c0);
                pd.d0 = m.p_lo & 7;
                pd.nv0 = std::max(0, std::min(pd.nck, m.nch0 - c0));
                pd.nv1 = (S & 1) ? std::max(0, std::min(pd.nck, m.nch1 - c0)) : 0;
                pd.tap0 = pd.nv0 > 0 ? m.tap0 + c0 : 0;
                pd.tap1 = pd.nv1 > 0 ? m.tap1 + c0 : 0;
                pieces.push_back(pd);
                c += 1.779 + 0.461 * pd.nck;
            }
        }
        if ((int)pieces.size() == piece_ptr[j]) {
            PieceDesc pd{0, 0, 0, 0, 1, 0, 0, 0};
            pieces.push_back(pd);
            c += 1.779 + 0.461;
        }
        piece_ptr[j + 1] = (int32_t)pieces.size();
        cost[j] = c;
        if (pieces.size() > (size_t)1 << 26) return DISCO_OK;
    }
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
    double total = 0.0;
    for (double c : cost) total += c;
    // contiguous latitude bands of equal cost, one per XCD: rows that share
    // input rows run close in time on the same L2
    std::vector<std::vector<int>> band(kNumXcd);
    {
        double acc = 0.0;
        for (int j = 0; j < nlat_out; ++j) {
            int k = (int)std::floor((acc + 0.5 * cost[j]) / total * kNumXcd);
            k = std::max(0, std::min(kNumXcd - 1, k));
            band[k].push_back(j);
            acc += cost[j];
        }
    }
    const int nqt = (D.nlon_out + kQ - 1) / kQ;
    info.assign(kInfoSize, 0);
    info[kInfoMagic] = 0x44495343;
    info[kInfoPiecePtr] = (int32_t)info.size();
    info.insert(info.end(), piece_ptr.begin(), piece_ptr.end());
    while (info.size() % 8) info.push_back(0);
    info[kInfoPieces] = (int32_t)info.size();
    info[kInfoNpieces] = (int32_t)pieces.size();
    const int* pp = reinterpret_cast<const int*>(pieces.data());
    info.insert(info.end(), pp, pp + pieces.size() * 8);
    info[kInfoItems] = (int32_t)info.size();
    int32_t off = 0;
    for (int k = 0; k < kNumXcd; ++k) {
        info[kInfoXcdOff + k] = off;
        for (int j : band[k])
            for (int qt = 0; qt < nqt; ++qt) {
                info.push_back(j);
                info.push_back(qt * kQ);
                info.push_back(piece_ptr[j]);
                info.push_back(piece_ptr[j + 1] - piece_ptr[j]);
            }
        info[kInfoXcdLen + k] = (int32_t)band[k].size() * nqt;
        off += info[kInfoXcdLen + k];
    }
    if (info.size() > (size_t)0x7fffffff) return DISCO_OK;
    return DISCO_OK;
}

namespace {

__device__ __forceinline__ floatx16 mfma(const bf16x8_t& a, const bf16x8_t& b, const floatx16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Weights into operand fragments: frag f = ((chunk*16 + ks)*(Co/32) + mt)*64 + lane holds
// w[co = mt*32 + lane%32][ci = chunk*32 + 2*ks + lane/32][k = 0..7] (zero for k >= K).
__global__ __launch_bounds__(256) void prep_weight_frags(const bf16_t* __restrict__ w,
                                                          u32x4* __restrict__ wf, int Ci, int Co,
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
    u32x4 o;
    o.x = v[0] | ((uint32_t)v[1] << 16);
    o.y = v[2] | ((uint32_t)v[3] << 16);
    o.z = v[4] | ((uint32_t)v[5] << 16);
    o.w = v[6] | ((uint32_t)v[7] << 16);
    wf[f] = o;
}

#define DISCO_VM_CASE(n) \
    case n: asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory"); break;

// Wait until at most n vector-memory operations of this wave are outstanding
// (n is wave-uniform; counts above 47 wait for everything).
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
        DISCO_VM_CASE(1) DISCO_VM_CASE(2) DISCO_VM_CASE(3) DISCO_VM_CASE(4) DISCO_VM_CASE(5)
        DISCO_VM_CASE(6) DISCO_VM_CASE(7) DISCO_VM_CASE(8) DISCO_VM_CASE(9) DISCO_VM_CASE(10)
        DISCO_VM_CASE(11) DISCO_VM_CASE(12) DISCO_VM_CASE(13) DISCO_VM_CASE(14) DISCO_VM_CASE(15)
        DISCO_VM_CASE(16) DISCO_VM_CASE(17) DISCO_VM_CASE(18) DISCO_VM_CASE(19) DISCO_VM_CASE(20)
        DISCO_VM_CASE(21) DISCO_VM_CASE(22) DISCO_VM_CASE(23) DISCO_VM_CASE(24) DISCO_VM_CASE(25)
        DISCO_VM_CASE(26) DISCO_VM_CASE(27) DISCO_VM_CASE(28) DISCO_VM_CASE(29) DISCO_VM_CASE(30)
        DISCO_VM_CASE(31) DISCO_VM_CASE(32) DISCO_VM_CASE(33) DISCO_VM_CASE(34) DISCO_VM_CASE(35)
        DISCO_VM_CASE(36) DISCO_VM_CASE(37) DISCO_VM_CASE(38) DISCO_VM_CASE(39) DISCO_VM_CASE(40)
        DISCO_VM_CASE(41) DISCO_VM_CASE(42) DISCO_VM_CASE(43) DISCO_VM_CASE(44) DISCO_VM_CASE(45)
        DISCO_VM_CASE(46) DISCO_VM_CASE(47)
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}
#undef DISCO_VM_CASE

__device__ __forceinline__ void barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void;

// 16-byte-per-lane DMA from global memory into LDS: lane l's 16 bytes land at
// lds + 16*l.  Written as inline asm on purpose: for the compiler's own
// global_load_lds it cannot tell which ring slot a pending transfer targets and
// waits for all of them (vmcnt(0)) before every later LDS read, which would
// serialise the ring.  These transfers are ordered explicitly instead: wait_vm
// on this wave's outstanding count, then a barrier.  The statement has no
// register outputs; M0 holds the LDS address, which is uniform across the
// wave (readfirstlane keeps it in a scalar register where the compiler's
// uniformity analysis loses track of that).
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
                 : "memory", "m0");
}

constexpr int kDmaWaves = 4;       // waves 0-3 only issue the DMA (one per SIMD)
constexpr int kWaves = 8;          // compute waves 4-11 (two per SIMD)
constexpr int kThreads = 64 * (kDmaWaves + kWaves);

__device__ __forceinline__ u32x4 bit_select(uint32_t m, const u32x4& a, const u32x4& b) {
    return (a & m) | (b & ~m);   // v_bfi_b32 per dword
}

// Record of one piece in the ring, written by the DMA waves when they issue it
// and read by every wave when it is consumed.
enum : int {
    kRecNck = 0xf,          // chunks (contraction piece)
    kRecHi = 1 << 4,        // window starts in the upper half of its 8-group (S = 1)
    kRecWeight = 1 << 5,    // weight piece; its index within the chunk in bits 6-7
    kRecLastC = 1 << 8,     // last contraction piece of the chunk: write the xk tile
    kRecEpi = 1 << 9,       // last piece of the work item (fused: write the output tile)
    kRecChunkShift = 16,    // channel chunk index in bits 16 and up
};

// XK = true: the contraction alone.  No weight pieces are streamed; the last
// piece of a channel chunk stores the chunk's xk tile (bf16) to
// y = xk[B, Ci, K, nlat_out, nlon_out] instead of feeding the GEMM.
template <int S, int CO, typename TY, bool XK = false>
__global__ __launch_bounds__(768, 1) void fused_mfma(
    const bf16_t* __restrict__ x, const u32x4* __restrict__ wfrag, const float* __restrict__ bias,
    TY* __restrict__ y, const int32_t* __restrict__ info, const u32x4* __restrict__ taps, int B,
    int Ci, int K, int nlat_in, int nlon_in, int nlat_out, int nlon_out) {
    constexpr int Q = kQ;
    constexpr int QW = Q / kWaves;                 // outputs per wave in the contraction
    constexpr int NBW = QW / 4;                    // 4-output blocks per wave
    constexpr int RS = row_stride(S);
    constexpr int NXI = x_instr(S);
    constexpr int NCI = NXI + tap_instr(S);        // DMA loads of a contraction piece
    constexpr int PWD = (NCI + kDmaWaves - 1) / kDmaWaves;   // loads per DMA wave per piece
    constexpr int SLOT = slot_size(S);
    constexpr int XSL = NXI * 64;
    constexpr int WM = CO / 32;                    // GEMM wave grid WM x WN, wave tile 32 x (Q/WN)
    constexpr int WN = kWaves / WM;
    constexpr int NT = Q / WN / 32;
    constexpr int NWI = kGemmSteps * (CO / 32);    // DMA loads of a weight piece
    constexpr int kNw = 16 / kGemmSteps;           // weight pieces per channel chunk
    constexpr int OS = sizeof(TY) == 4 ? 132 : 136;   // output tile row stride (elements)
    constexpr int EPC = 16 / (int)sizeof(TY);         // output elements per 16-byte store
    constexpr int CPR = Q / EPC;                      // 16-byte stores per output row
    constexpr int kStoreThreads = 64 * kWaves;
    constexpr int NST = CO * CPR / kStoreThreads;     // stores per store thread per item
    static_assert(NWI <= kDmaWaves * PWD && NWI * 64 <= SLOT, "weight piece layout");
    static_assert(WM * WN == kWaves && NT >= 1, "GEMM wave grid");
    static_assert(CO * OS * (int)sizeof(TY) <= Q * kXkStride * 2, "output tile fits the xk tile");
    static_assert(QW % 8 == 0 && NBW % 2 == 0, "wave output range keeps 8-alignment");
    static_assert(NST * kStoreThreads == CO * CPR, "store split");
    static_assert(2 * PWD <= 63, "vmcnt range");
    static_assert(kDmaWaves * PWD == NCI || NCI - kDmaWaves >= NXI, "repeated loads are tap loads");
    static_assert(!XK || (sizeof(TY) == 2 && 32 * 16 == 64 * kWaves), "xk store split");

    // fused: xk tile [q][(ci, k)]; XK: transposed tile [(k, ci)][q]
    __shared__ __attribute__((aligned(16))) bf16_t xk_lds[XK ? 256 * kXkTStride : Q * kXkStride];
    __shared__ __attribute__((aligned(16))) u32x4 ring[kRing][SLOT];
    __shared__ int4 rec_lds[kRing];
    __shared__ float bias_lds[CO];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const bool dma_wave = wv < kDmaWaves;
    const int wave = dma_wave ? wv : wv - kDmaWaves;   // index among the DMA / compute waves
    const int lg = lane >> 5;
    const int l32 = lane & 31;
    const int wm = wave / WN, wn = wave % WN;

    const int xcd = blockIdx.x % kNumXcd;
    const int r = blockIdx.x / kNumXcd;
    const int nwg = gridDim.x / kNumXcd;
    const int xlen = info[kInfoXcdLen + xcd];
    const int my_items = xlen > r ? (xlen - r + nwg - 1) / nwg : 0;   // items r, r + nwg, ...
    const int total = B * my_items;
    if (total == 0) return;
    const int nchunks = Ci / 32;
    const size_t plane_in = (size_t)nlat_in * nlon_in;
    const size_t plane_out = (size_t)nlat_out * nlon_out;

    for (int c = tid; c < CO; c += kThreads) bias_lds[c] = bias ? bias[c] : 0.0f;

    floatx16 g[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) g[c][e] = 0.0f;
    floatx16 acc[NBW];
#pragma unroll
    for (int n = 0; n < NBW; ++n)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[n][e] = 0.0f;

    // ---------------- DMA waves: the issue cursor ----------------
    // (all of its state is wave-uniform; only waves 0-3 touch it)
    const int4* items = reinterpret_cast<const int4*>(info + info[kInfoItems]) + info[kInfoXcdOff + xcd];
    const PieceDesc* pdesc = reinterpret_cast<const PieceDesc*>(info + info[kInfoPieces]);
    const uint32_t ring_base =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void*)&ring[0][0]);
    const bool short_rows = 8 * RS > nlon_in;   // a strip may wrap more than once
    int lch[PWD], lgr[PWD];                     // this lane's slot in the wave's strip loads
#pragma unroll
    for (int m = 0; m < PWD; ++m) {
        const int sl = 64 * (wave + kDmaWaves * m) + lane;
        int ci = sl / RS, grp = sl - (sl / RS) * RS;
        if (ci >= 32) { ci = 0; grp = 1 << 20; }   // padding slot: never valid
        lch[m] = ci * (int)plane_in;
        lgr[m] = grp;
    }
    // cursor: item k of this workgroup's list, batch entry b, chunk cc, piece pi
    int c_k = 0, c_b = 0, c_cc = 0, c_pi = 0, c_t = 0;
    int4 c_it = items[r];                           // (j, q0, first piece, pieces)
    int4 c_nx = items[r + (my_items > 1 ? nwg : 0)];   // the next item (prefetched)
    const bf16_t* c_xb = x;                         // channel chunk base of (b, cc)
    PieceDesc pdn;                                  // descriptor of the piece at the cursor
    pdn = pdesc[c_it.z];
    auto advance = [&]() {
        if (++c_pi == c_it.w + (XK ? 0 : kNw)) {
            c_pi = 0;
            if (++c_cc == nchunks) {
                c_cc = 0;
                ++c_t;
                if (++c_k == my_items) { c_k = 0; ++c_b; }
                c_it = c_nx;
                int k2 = c_k + 1, b2 = c_b;
                if (k2 == my_items) { k2 = 0; ++b2; }
                if (b2 < B) c_nx = items[r + k2 * nwg];
            }
            c_xb = x + ((size_t)c_b * Ci + (size_t)c_cc * 32) * plane_in;
        }
        if (c_t < total && c_pi < c_it.w) pdn = pdesc[c_it.z + c_pi];   // used at the next issue
    };
    // issue the piece at the cursor into ring slot `slot` (PWD loads per DMA
    // wave; loads without work repeat a valid load) and publish its record
    auto issue = [&](int slot) -> int {
        const uint32_t dst = ring_base + (uint32_t)slot * (SLOT * 16);
        int rec;
        if (!XK && c_pi >= c_it.w) {
            const int wp = c_pi - c_it.w;
            const u32x4* src = wfrag + ((size_t)(c_cc * 16 + wp * kGemmSteps) * (CO / 32)) * 64;
#pragma unroll
            for (int m = 0; m < PWD; ++m) {
                int i = wave + kDmaWaves * m;
                if (i >= NWI) i = wave + kDmaWaves * ((NWI - 1 - wave) / kDmaWaves);   // repeat
                dma16(src + 64 * i + lane, dst + i * 1024);
            }
            rec = kRecWeight | (wp << 6) |
                  (wp == kNw - 1 && c_cc == nchunks - 1 ? kRecEpi : 0);
        } else {
            const bf16_t* xrow = c_xb + pdn.xoff;
            int u0 = S * c_it.y + pdn.uoff;
            if (u0 >= nlon_in) u0 -= nlon_in;
            const int ngrp = piece_groups(S, pdn.nck);
#pragma unroll
            for (int m = 0; m < PWD; ++m) {
                const int i0 = wave + kDmaWaves * m;
                if (i0 < NXI) {
                    int gx = u0 + 8 * lgr[m];
                    if (short_rows) gx %= nlon_in;
                    else gx -= gx >= nlon_in ? nlon_in : 0;
                    const bf16_t* src = lgr[m] < ngrp ? xrow + lch[m] + gx : xrow + u0;
                    dma16(src, dst + i0 * 1024);
                } else {
                    // loads past the piece's end repeat this wave's previous tap load
                    const int i = i0 >= NCI ? i0 - kDmaWaves : i0;
                    const int f = i - NXI;              // chunk f / classes, class f % classes
                    const int kk = (S & 1) ? (f >> 1) : f;
                    const int cls = (S & 1) ? (f & 1) : 0;
                    const int nv = cls ? pdn.nv1 : pdn.nv0;
                    const int fr = kk < nv ? (cls ? pdn.tap1 : pdn.tap0) + kk : 0;   // 0: zero fragment
                    dma16(taps + (size_t)fr * 64 + lane, dst + i * 1024);
                }
            }
            const bool last = c_pi == c_it.w - 1;
            rec = pdn.nck | (pdn.d0 >= 4 ? kRecHi : 0) | (last ? kRecLastC : 0) |
                  (XK && last && c_cc == nchunks - 1 ? kRecEpi : 0) | (c_cc << kRecChunkShift);
        }
        if (wave == 0 && lane == 0) rec_lds[slot] = make_int4(rec, c_b, c_it.x, c_it.y);
        return rec;
    };

    if (dma_wave) {
        // ================= DMA waves =================
        // prologue: three pieces in flight (a fused work item has at least
        // 1 + kNw pieces; XK: up to three)
        uint32_t epi_mask = 0;     // ring slots whose piece ends a work item
        uint32_t lastc_mask = 0;   // XK: ring slots whose piece ends a channel chunk
        for (int k = 0; k < kRing - 1 && (!XK || c_t < total); ++k) {
            const int rec = issue(k);
            if (rec & kRecEpi) epi_mask |= 1u << k;
            if (XK && (rec & kRecLastC)) lastc_mask |= 1u << k;
            advance();
        }
        bool more = c_t < total;
        __syncthreads();   // bias_lds, rec_lds of the first pieces
        int done = 0;
        for (int seq = 0;; ++seq) {
            // piece seq is complete once only the two later pieces' loads remain
            if (more) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PWD) : "memory");
            else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            barrier();   // piece seq is in LDS for every wave; slot (seq + 3) % 4 is free
            const int slot = seq & (kRing - 1);
            if (more) {
                const int ns = (seq + kRing - 1) & (kRing - 1);
                const int rec = issue(ns);
                if (rec & kRecEpi) epi_mask |= 1u << ns;
                if (XK && (rec & kRecLastC)) lastc_mask |= 1u << ns;
                advance();
                more = c_t < total;
            }
            if (XK && (lastc_mask & (1u << slot))) {
                // the compute waves write the xk tile before this barrier and
                // store it after
                lastc_mask &= ~(1u << slot);
                barrier();
            }
            if (epi_mask & (1u << slot)) {
                // fused: the compute waves write the output tile between two barriers
                epi_mask &= ~(1u << slot);
                if (!XK) {
                    barrier();
                    barrier();
                }
                if (++done == total) break;
            }
        }
        return;
    }

    // ================= compute waves =================
    __syncthreads();   // bias_lds, rec_lds of the first pieces
    // The compute side walks the stream through the records; it ends with the
    // epilogue of the last work item.
    int done = 0;
    for (int seq = 0;; ++seq) {
        barrier();   // piece seq is in LDS for every wave
        const int slot = seq & (kRing - 1);
        const int4 rq = rec_lds[slot];
        const int rf = __builtin_amdgcn_readfirstlane(rq.x);
        if (!(rf & kRecWeight)) {
            // ---- contraction piece ----        } else if (!(rf & kRecWeight)) {
            // ---- contraction piece ----
            const bf16_t* xs = reinterpret_cast<const bf16_t*>(ring[slot]);
            const u32x4* ts = ring[slot] + XSL;
            const int row = l32 * RS + (S * QW * wave) / 8 + lg;
            const int nck = rf & kRecNck;
            // S = 1: block n of chunk kk reads staged group 2*kk + n/2, one more for
            // odd n when the window starts in the upper half of its 8-group; class-0
            // taps for even blocks, class 1 for odd.  S = 2: group 2*kk + n, class 0.
            // Chunks beyond a class's band hold the zero fragment.
            const uint32_t hm = (rf & kRecHi) ? 0xffffffffu : 0u;
            for (int kk = 0; kk < nck; ++kk) {
                constexpr int NV = S == 1 ? NBW / 2 + 1 : NBW;
                u32x4 f[NV];
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    f[v] = *reinterpret_cast<const u32x4*>(xs + 8 * (row + 2 * kk + v));
                const int f0 = (S & 1) ? 2 * kk : kk;
                const bf16x8_t a0 = as_bf16x8(ts[64 * f0 + lane]);
                if (S == 1) {
                    const bf16x8_t a1 = as_bf16x8(ts[64 * (f0 + 1) + lane]);
#pragma unroll
                    for (int m = 0; m < NBW / 2; ++m) {
                        acc[2 * m] = mfma(a0, as_bf16x8(f[m]), acc[2 * m]);
                        acc[2 * m + 1] =
                            mfma(a1, as_bf16x8(bit_select(hm, f[m + 1], f[m])), acc[2 * m + 1]);
                    }
                } else {
#pragma unroll
                    for (int n = 0; n < NBW; ++n) acc[n] = mfma(a0, as_bf16x8(f[n]), acc[n]);
                }
            }
            if (XK && (rf & kRecLastC)) {
                // the chunk's contraction is complete: transposed xk tile
                // (bf16) -> LDS, row k * 32 + ci, 4 outputs per 8-byte write
#pragma unroll
                for (int n = 0; n < NBW; ++n) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float4v v4 = {acc[n][e], acc[n][4 + e], acc[n][8 + e], acc[n][12 + e]};
                        const u32x2 pk =
                            __builtin_bit_cast(u32x2, __builtin_convertvector(v4, bf16x4_t));
                        *reinterpret_cast<u32x2*>(xk_lds + ((4 * lg + e) * 32 + l32) * kXkTStride +
                                                  wave * QW + 4 * n) = pk;
                    }
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[n][e] = 0.0f;
                }
                barrier();   // the tile is complete
                // store thread st writes 16 bytes (8 outputs) of row (k, st / 16)
                // per k; outputs past the row's end are not written
                const int eb = __builtin_amdgcn_readfirstlane(rq.y);
                const int ej = __builtin_amdgcn_readfirstlane(rq.z);
                const int eq0 = __builtin_amdgcn_readfirstlane(rq.w);
                const int cc = rf >> kRecChunkShift;
                const int st = tid - 64 * kDmaWaves;
                const int ci = st >> 4, q = eq0 + 8 * (st & 15);
                const bf16_t* os = xk_lds + ci * kXkTStride + 8 * (st & 15);
                TY* ob = y + ((size_t)(eb * Ci + cc * 32 + ci) * K) * plane_out +
                         (size_t)ej * nlon_out + q;
                if (q < nlon_out) {
                    for (int k = 0; k < K; ++k)
                        *reinterpret_cast<u32x4*>(ob + (size_t)k * plane_out) =
                            *reinterpret_cast<const u32x4*>(os + k * 32 * kXkTStride);
                }
                if (rf & kRecEpi) {
                    if (++done == total) break;
                }
            } else if (!XK && (rf & kRecLastC)) {
                // the chunk's contraction is complete: xk tile (bf16) -> LDS
#pragma unroll
                for (int n = 0; n < NBW; ++n) {
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        const int ql = wave * QW + 4 * n + qq;
                        const float4v v4 = {acc[n][4 * qq + 0], acc[n][4 * qq + 1],
                                            acc[n][4 * qq + 2], acc[n][4 * qq + 3]};
                        const u32x2 pk =
                            __builtin_bit_cast(u32x2, __builtin_convertvector(v4, bf16x4_t));
                        *reinterpret_cast<u32x2*>(xk_lds + ql * kXkStride + l32 * 8 + 4 * lg) = pk;
                    }
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[n][e] = 0.0f;
                }
            }
        } else {
            // ---- weight piece: kGemmSteps k-steps of the channel/basis GEMM ----
            const int wp = (rf >> 6) & 3;
            const u32x4* ws = ring[slot];
#pragma unroll
            for (int ks = 0; ks < kGemmSteps; ++ks) {
                const int kg = wp * kGemmSteps + ks;
                const bf16x8_t af = as_bf16x8(ws[(ks * (CO / 32) + wm) * 64 + lane]);
#pragma unroll
                for (int c = 0; c < NT; ++c) {
                    const int ql = wn * (Q / WN) + c * 32 + l32;
                    const bf16x8_t bf =
                        *reinterpret_cast<const bf16x8_t*>(xk_lds + ql * kXkStride + kg * 16 + 8 * lg);
                    g[c] = mfma(af, bf, g[c]);
                }
            }
            if (rf & kRecEpi) {
                // ---- epilogue: the item's output tile, transposed through LDS ----
                const int eb = __builtin_amdgcn_readfirstlane(rq.y);
                const int ej = __builtin_amdgcn_readfirstlane(rq.z);
                const int eq0 = __builtin_amdgcn_readfirstlane(rq.w);
                barrier();   // every wave is done reading the xk tile
                // lane base pointers; every element below is a compile-time offset
                TY* ot = reinterpret_cast<TY*>(xk_lds) + (wm * 32 + 4 * lg) * OS + wn * (Q / WN) + l32;
                const float* bl = bias_lds + wm * 32 + 4 * lg;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int cr = 8 * (e >> 2) + (e & 3);   // row within the lane base
                    const float bv = bl[cr];
#pragma unroll
                    for (int c = 0; c < NT; ++c) {
                        const float v = g[c][e] + bv;
                        if constexpr (sizeof(TY) == 4) ot[cr * OS + c * 32] = v;
                        else ot[cr * OS + c * 32] = f32_to_bf16(v);
                        g[c][e] = 0.0f;
                    }
                }
                barrier();
                {
                    // store thread st stores 16-byte column group st % CPR of rows
                    // st / CPR + k * (kStoreThreads / CPR); columns past the end
                    // rewrite the row's last valid 16 bytes with the same data
                    const int st = tid - 64 * kDmaWaves;
                    const int qc = min((st % CPR) * EPC, ((nlon_out - eq0 - 1) / EPC) * EPC);
                    const TY* os = reinterpret_cast<const TY*>(xk_lds) + (st / CPR) * OS + qc;
                    TY* yb = y + ((size_t)eb * CO + st / CPR) * plane_out + (size_t)ej * nlon_out +
                             eq0 + qc;
#pragma unroll
                    for (int k = 0; k < NST; ++k)
                        *reinterpret_cast<u32x4*>(yb + (size_t)k * (kStoreThreads / CPR) * plane_out) =
                            *reinterpret_cast<const u32x4*>(os + k * (kStoreThreads / CPR) * OS);
                }
                if (++done == total) break;
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace

// Scratch of the no-allocation fused entry point: the direct kernel's weight
// fragments live here instead of in stream-ordered workspace.  Host code
// never uses the array's name as an address: each device's copy is looked up
// once with hipGetSymbolAddress (noalloc_scratch) and that address is passed
// to the kernels.  Every call on a device shares its copy; calls that overlap
// on one device race.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

int noalloc_scratch(void** ptr, size_t* bytes) {
    static std::mutex mu;
    static void* addr[64] = {nullptr};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return set_error(DISCO_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    }
    if (dev < 0 || dev >= 64) return set_error(DISCO_EUNSUPPORTED, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return set_error(DISCO_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s",
                             dev, hipGetErrorString(e));
        }
        addr[dev] = p;
    }
    *ptr = addr[dev];
    *bytes = kNoAllocScratchBytes;
    return DISCO_OK;
}

// Bytes of weight fragments the direct matrix-core kernel needs.
size_t fused_mfma_frag_bytes(int Ci, int Co) {
    return (size_t)(Ci / 32) * 16 * (Co / 32) * 64 * sizeof(u32x4);
}

int try_launch_fused_mfma(const disco_psi* psi, const void* x, const void* w, const float* bias,
                          void* y, int y_dtype, int B, int Ci, int Co, int groups, hipStream_t st,
                          int* rc, void* frag_ws, size_t frag_ws_bytes) {
    const DevPsi& d = psi->dev;
    const HostPsi& h = psi->host;
    const disco_psi_desc& D = h.desc;
    if (!d.mfma_ok || groups != 1 || Ci % 32 != 0 || (Co != 128 && Co != 64) || h.K > 8) return 0;
    const int S = h.stride;
    if (S != 1 && S != 2) return 0;
    // 16-byte loads of x and 16-byte stores of y rows
    const int epc = y_dtype == DISCO_F32 ? 4 : 8;
    if ((reinterpret_cast<uintptr_t>(x) & 15) != 0 || (reinterpret_cast<uintptr_t>(y) & 15) != 0 ||
        D.nlon_out % epc != 0)
        return 0;
    // channel offsets of one 32-channel chunk are 32-bit
    if ((int64_t)D.nlat_in * D.nlon_in * 32 >= ((int64_t)1 << 31)) return 0;
    if (B <= 0) return 0;
    const int32_t* dinfo = d.mfma_row_info;
    const u32x4* taps = static_cast<const u32x4*>(d.mfma_taps);

    // weight fragments: the caller's fixed scratch, or stream-ordered workspace
    const size_t nfrag = (size_t)(Ci / 32) * 16 * (Co / 32) * 64;
    void* wsp = nullptr;
    // without the caller's scratch: the handle's workspace (stream-ordered
    // memory while a graph is captured)
    WorkspaceLease lease(frag_ws != nullptr ? nullptr : psi, nfrag * sizeof(u32x4), st);
    if (lease.error() != DISCO_OK) {
        *rc = lease.error();
        return 1;
    }
    const bool own_ws = frag_ws == nullptr && lease.ptr() == nullptr;
    if (frag_ws != nullptr) {
        if (nfrag * sizeof(u32x4) > frag_ws_bytes) {
            *rc = set_error(DISCO_EINVAL, "the weight fragments need %zu bytes of scratch; only "
                            "%zu are available", nfrag * sizeof(u32x4), frag_ws_bytes);
            return 1;
        }
        wsp = frag_ws;
    } else if (!own_ws) {
        wsp = lease.ptr();
    } else {
        hipError_t e = hipMallocAsync(&wsp, nfrag * sizeof(u32x4), st);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            *rc = set_error(e == hipErrorOutOfMemory ? DISCO_ENOMEM : DISCO_EHIP,
                            "hipMallocAsync for the weight fragments failed: %s",
                            hipGetErrorString(e));
            return 1;
        }
    }
    u32x4* wf = static_cast<u32x4*>(wsp);
    {
        KernelTimer timer("prep_weight_frags", st);
        hipLaunchKernelGGL(prep_weight_frags, dim3((unsigned)((nfrag + 255) / 256)), dim3(256), 0,
                           st, static_cast<const bf16_t*>(w), wf, Ci, Co, h.K);
    }
    const bf16_t* X = static_cast<const bf16_t*>(x);
    // one persistent workgroup per CU: 32 per XCD
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    (void)hipGetLastError();
    const int per_xcd = std::max(1, ncu / kNumXcd);
    dim3 grid((unsigned)(kNumXcd * per_xcd));
#define DISCO_FM(SS, CC, TT)                                                                 \
    hipLaunchKernelGGL((fused_mfma<SS, CC, TT>), grid, dim3(kThreads), 0, st, X, wf, bias, (TT*)y, \
                       dinfo, taps, B, Ci, h.K, D.nlat_in, D.nlon_in, D.nlat_out, D.nlon_out)
    {
    KernelTimer timer("fused_mfma", st);
    const bool f32 = y_dtype == DISCO_F32;
    if (Co == 128) {
        if (S == 1) { if (f32) DISCO_FM(1, 128, float); else DISCO_FM(1, 128, bf16_t); }
        else        { if (f32) DISCO_FM(2, 128, float); else DISCO_FM(2, 128, bf16_t); }
    } else {
        if (S == 1) { if (f32) DISCO_FM(1, 64, float); else DISCO_FM(1, 64, bf16_t); }
        else        { if (f32) DISCO_FM(2, 64, float); else DISCO_FM(2, 64, bf16_t); }
    }
    }
#undef DISCO_FM
    hipError_t le = hipGetLastError();
    hipError_t fe = own_ws ? hipFreeAsync(wsp, st) : hipSuccess;
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

bool contract_mfma_ok(const disco_psi* psi, const void* x, const void* xk, int B, int C) {
    const DevPsi& d = psi->dev;
    const HostPsi& h = psi->host;
    const disco_psi_desc& D = h.desc;
    if (!d.mfma_ok || C % 32 != 0 || h.K > 8 || B <= 0) return false;
    if (h.stride != 1 && h.stride != 2) return false;
    // 16-byte loads of x rows and 16-byte stores of xk rows
    if ((reinterpret_cast<uintptr_t>(x) & 15) != 0 || (reinterpret_cast<uintptr_t>(xk) & 15) != 0 ||
        D.nlon_out % 8 != 0)
        return false;
    // channel offsets of one 32-channel chunk are 32-bit
    return (int64_t)D.nlat_in * D.nlon_in * 32 < ((int64_t)1 << 31);
}

int try_launch_contract_mfma(const disco_psi* psi, const void* x, void* xk, int B, int C,
                             hipStream_t st, int* rc) {
    const DevPsi& d = psi->dev;
    const HostPsi& h = psi->host;
    const disco_psi_desc& D = h.desc;
    if (!contract_mfma_ok(psi, x, xk, B, C)) return 0;
    const int S = h.stride;
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    (void)hipGetLastError();
    const int per_xcd = std::max(1, ncu / kNumXcd);
    dim3 grid((unsigned)(kNumXcd * per_xcd));
    const bf16_t* X = static_cast<const bf16_t*>(x);
    bf16_t* XK = static_cast<bf16_t*>(xk);
    const int32_t* dinfo = d.mfma_row_info;
    const u32x4* taps = static_cast<const u32x4*>(d.mfma_taps);
#define DISCO_CM(SS)                                                                             \
    hipLaunchKernelGGL((fused_mfma<SS, 128, bf16_t, true>), grid, dim3(kThreads), 0, st, X,       \
                       nullptr, nullptr, XK, dinfo, taps, B, C, h.K, D.nlat_in, D.nlon_in,         \
                       D.nlat_out, D.nlon_out)
    {
        KernelTimer timer("contract_mfma", st);
        if (S == 1) DISCO_CM(1);
        else DISCO_CM(2);
    }
#undef DISCO_CM
    hipError_t le = hipGetLastError();
    if (le != hipSuccess) {
        *rc = set_error(DISCO_EHIP, "contraction (matrix cores) launch failed: %s",
                        hipGetErrorString(le));
        return 1;
    }
    *rc = DISCO_OK;
    return 1;
}

}  // namespace disco
