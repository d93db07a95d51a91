// Device helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace disco {

typedef uint16_t bf16_t;   // raw bfloat16 storage

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// float -> bfloat16, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>(0x7fc0u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

__device__ __forceinline__ float load_f(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_f(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }

__device__ __forceinline__ void store_f(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_f(bf16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }

// Wave-uniform value (lets the compiler keep it in a scalar register).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS: lane L writes
// lds_addr + 16 L (global_load_lds_dwordx4, LDS address in M0).  No register
// results: completion is tracked by the caller's vmcnt waits.
__device__ __forceinline__ void dma_lds16(const void* src, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
                 : "memory", "m0");
}

// Wait until at most N vector memory operations of this wave are outstanding
// (s_waitcnt with the export and LDS/scalar counts left at their maxima; the
// builtin, unlike inline asm, is seen by the compiler's own wait placement).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace disco
