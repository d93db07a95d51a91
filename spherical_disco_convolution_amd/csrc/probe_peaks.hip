// Micro-benchmarks of the gfx950 rates the roofline figures are priced
// against: HBM copy and read bandwidth, dense bf16 matrix-core rate and LDS
// read bandwidth.  Built into libdisco_probe.so, separate from the library:
// the benchmark calls them to confirm on the machine the published peaks it
// divides by.  Each probe times its own launches with HIP events on the null
// stream and returns milliseconds.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// dst[i] = src[i], 16 bytes per lane per step, grid-stride
__global__ __launch_bounds__(256) void copy16(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                              size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// XOR of all 16-byte words of src (read-only stream), one word per workgroup
// written to out so that the loads stay live
__global__ __launch_bounds__(256) void read16(const uint4* __restrict__ src, size_t n,
                                              uint32_t* __restrict__ out) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    uint4 acc = make_uint4(0, 0, 0, 0);
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const uint4 v = src[i];
        acc.x ^= v.x;
        acc.y ^= v.y;
        acc.z ^= v.z;
        acc.w ^= v.w;
    }
    const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (r == 0x9e3779b9u) out[blockIdx.x] = r;   // practically never taken
}

// Four independent v_mfma_f32_32x32x16_bf16 chains per wave.
__global__ __launch_bounds__(256) void mfma_chain(float* __restrict__ out, int iters) {
    bf16x8_t a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1.0f / (float)(1 + ((threadIdx.x + e) & 7)));
        b[e] = (__bf16)(1.0f / (float)(2 + ((threadIdx.x * 3 + e) & 7)));
    }
    floatx16 c0, c1, c2, c3;
#pragma unroll
    for (int e = 0; e < 16; ++e) c0[e] = c1[e] = c2[e] = c3[e] = 0.0f;
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Conflict-free 16-byte LDS reads: each wave reads 1 KB contiguous per step.
// 64 KB of LDS per workgroup: at most two workgroups per compute unit.
constexpr int kLdsWords = 4096;   // 64 KB of 16-byte words
__global__ __launch_bounds__(256) void lds_read(uint32_t* __restrict__ out, int iters) {
    __shared__ uint4 buf[kLdsWords];
    for (int i = threadIdx.x; i < kLdsWords; i += blockDim.x)
        buf[i] = make_uint4(i, i * 3u, i * 5u, i * 7u);
    __syncthreads();
    uint4 acc = make_uint4(0, 0, 0, 0);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int idx = wave * 1024 + lane;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint4 v = buf[(idx + 64 * u) & (kLdsWords - 1)];
            acc.x ^= v.x;
            acc.y ^= v.y;
            acc.z ^= v.z;
            acc.w ^= v.w;
        }
        idx += 512;   // every iteration reads new addresses
    }
    const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (r == 0x9e3779b9u) out[blockIdx.x] = r;
}

// 16-byte LDS reads in a given lane pattern (each wave reads 1 KB per
// instruction): mode 0 contiguous (lane l at 16 l); mode 1 and 2 rows of
// 128 bytes, one per lane (row l & 31, lane halves 4 KB apart), at 16-byte
// piece (l & 7) (mode 1) or ((l >> 1) & 7) (mode 2) of the row.  On a 64-bank
// LDS with 16-lane phases mode 1 has two-way conflicts and mode 2 none; with
// 32 banks and 8-lane phases it is the other way round.
__global__ __launch_bounds__(256) void lds_pattern(uint32_t* __restrict__ out, int iters, int mode) {
    __shared__ uint4 buf[kLdsWords];
    for (int i = threadIdx.x; i < kLdsWords; i += blockDim.x)
        buf[i] = make_uint4(i, i * 3u, i * 5u, i * 7u);
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, lg = lane >> 5;
    int base;
    if (mode == 0) base = lane;
    else if (mode == 1) base = lg * 256 + l32 * 8 + (l32 & 7);
    else base = lg * 256 + l32 * 8 + ((l32 >> 1) & 7);
    base += wave * 512;
    uint4 acc = make_uint4(0, 0, 0, 0);
    int off = 0;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            // in bounds: base < 2048, off + 512 u < 2048 before the mask
            const uint4 v = buf[(base + ((off + 512 * u) & 2047)) & (kLdsWords - 1)];
            acc.x ^= v.x;
            acc.y ^= v.y;
            acc.z ^= v.z;
            acc.w ^= v.w;
        }
        off += 64;
    }
    const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (r == 0x9e3779b9u) out[blockIdx.x] = r;
}

template <typename F>
int timed(F launch, int reps, float* ms) {
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -4;
    launch();   // warm-up
    if (hipEventRecord(e0, nullptr) != hipSuccess) return -4;
    for (int r = 0; r < reps; ++r) launch();
    if (hipEventRecord(e1, nullptr) != hipSuccess) return -4;
    if (hipEventSynchronize(e1) != hipSuccess) return -4;
    float t = 0.0f;
    (void)hipEventElapsedTime(&t, e0, e1);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    *ms = t / (float)reps;
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int grid_for(int per_cu) {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    return ncu * per_cu;
}

}  // namespace

extern "C" {

// Device-to-device copy of `bytes` (a multiple of 16) from src to dst, both
// device buffers of at least that size.  *ms: average time per copy.
int probe_hbm_copy(void* dst, const void* src, size_t bytes, int reps, float* ms) {
    if (!dst || !src || !ms || bytes % 16 || reps < 1) return -1;
    const size_t n = bytes / 16;
    const int grid = grid_for(8);
    return timed([&] {
        hipLaunchKernelGGL(copy16, dim3(grid), dim3(256), 0, nullptr, static_cast<uint4*>(dst),
                           static_cast<const uint4*>(src), n);
    }, reps, ms);
}

// Read-only stream over `bytes` (a multiple of 16) of src; scratch: a device
// buffer of at least 4 bytes per workgroup (grid = 8 per compute unit).
int probe_hbm_read(const void* src, size_t bytes, void* scratch, int reps, float* ms) {
    if (!src || !scratch || !ms || bytes % 16 || reps < 1) return -1;
    const size_t n = bytes / 16;
    const int grid = grid_for(8);
    return timed([&] {
        hipLaunchKernelGGL(read16, dim3(grid), dim3(256), 0, nullptr,
                           static_cast<const uint4*>(src), n, static_cast<uint32_t*>(scratch));
    }, reps, ms);
}

// Dense bf16 matrix-core rate: `per_cu` workgroups of four waves per compute
// unit, each wave issuing 4 * iters v_mfma_f32_32x32x16_bf16.  out: device
// buffer of 256 * grid floats.  *flop: floating-point operations per launch.
int probe_mfma_bf16(float* out, int per_cu, int iters, int reps, float* ms, double* flop) {
    if (!out || !ms || !flop || per_cu < 1 || iters < 1 || reps < 1) return -1;
    const int grid = grid_for(per_cu);
    *flop = (double)grid * 4 /* waves */ * 4 /* chains */ * iters * (2.0 * 32 * 32 * 16);
    return timed([&] {
        hipLaunchKernelGGL(mfma_chain, dim3(grid), dim3(256), 0, nullptr, out, iters);
    }, reps, ms);
}

// LDS read bandwidth: `per_cu` workgroups of four waves per compute unit, each
// wave reading 8 KB per iteration.  scratch: 4 bytes per workgroup.
// *bytes: LDS bytes read per launch.
int probe_lds_read(void* scratch, int per_cu, int iters, int reps, float* ms, double* bytes) {
    if (!scratch || !ms || !bytes || per_cu < 1 || iters < 1 || reps < 1) return -1;
    const int grid = grid_for(per_cu);
    *bytes = (double)grid * 4 * iters * 8 * 64 * 16.0;
    return timed([&] {
        hipLaunchKernelGGL(lds_read, dim3(grid), dim3(256), 0, nullptr,
                           static_cast<uint32_t*>(scratch), iters);
    }, reps, ms);
}

// LDS read time for one lane pattern of lds_pattern (modes 0, 1, 2); two
// workgroups of four waves per compute unit, each wave reading 8 KB per
// iteration.  scratch: 4 bytes per workgroup.
int probe_lds_pattern(void* scratch, int mode, int iters, int reps, float* ms, double* bytes) {
    if (!scratch || !ms || !bytes || mode < 0 || mode > 2 || iters < 1 || reps < 1) return -1;
    const int grid = grid_for(2);
    *bytes = (double)grid * 4 * iters * 8 * 64 * 16.0;
    return timed([&] {
        hipLaunchKernelGGL(lds_pattern, dim3(grid), dim3(256), 0, nullptr,
                           static_cast<uint32_t*>(scratch), iters, mode);
    }, reps, ms);
}

// Compute units of the current device (0 on error).
int probe_num_cus(void) {
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return ncu;
}

}  // extern "C"
