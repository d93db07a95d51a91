// Internal declarations shared by the host builder, the C-ABI layer and the
// HIP kernel launchers.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/disco.h"

namespace disco {

// ---------------------------------------------------------------------------
// Errors
// ---------------------------------------------------------------------------
int set_error(int code, const char* fmt, ...);   // records message, returns code
void clear_error();

// ---------------------------------------------------------------------------
// Host form of Psi (float64)
// ---------------------------------------------------------------------------
// One support window: the input row `lat` contributes longitudes
// p = (p_lo + t) mod nlon_in for t in [0, width) to one output row.
struct Window {
    int32_t lat;
    int32_t p_lo;
    int32_t width;
    int64_t val_off;   // offset (in support points) into the window-ordered values
};

struct HostPsi {
    disco_psi_desc desc;
    double cutoff;
    int32_t nr, nphi, K, stride;
    // canonical CSR (sorted by (lat, lon) within each output row)
    std::vector<int64_t> row_ptr;
    std::vector<int32_t> in_lat, lon_off;
    std::vector<double> vals;            // [nnz, K]
    int64_t nnz_nonzero = 0;
    // window form: per output row, windows sorted by input row
    std::vector<int64_t> win_ptr;        // [nlat_out + 1]
    std::vector<Window> windows;
    std::vector<double> win_vals;        // [nnz, K] in window order (t ascending)
};

// Validates the description and builds the host form.  Returns DISCO_OK or an
// error code (message recorded).
int build_host_psi(const disco_psi_desc& desc, HostPsi& out);

// Longitude-spectral tables (spectral_host.cpp), built for stride-1 layers
// whose longitude count N is even, at most kSpecMaxN, with N/2 a product of
// 2, 3 and 5, and K <= 8.  psih: [nwin][K][MP] bf16 (re, im) pairs in 32-bit
// words (real part low), Psi_hat of each window, followed by 32 zero words;
// radix: the plan of the N/2-point transform.  *mp = 0 when the layer
// does not qualify.
constexpr int kSpecMaxN = 1800;   // N/2 <= 900 bounds the transform butterflies per lane
constexpr int kSpecMaxRadix = 12;
int spectral_plan(int n, int32_t* radix, int32_t* nrad);
int build_spectral_tables(const HostPsi& h, std::vector<uint32_t>& psih, int32_t* radix,
                          int32_t* nrad, int32_t* mp);

// ---------------------------------------------------------------------------
// Device form of Psi
// ---------------------------------------------------------------------------
struct DevWindow {            // 16 bytes, one per (output row, input row) window
    int32_t lat;
    int32_t p_lo;
    int32_t width;
    int32_t val_off;          // in points; values at val_off*KP
};

struct DevPsi {
    int device = -1;
    int32_t KP = 0;               // K padded for the vector kernels
    int32_t max_row_points = 0;   // max support points of one output row
    int32_t max_width = 0;        // widest window
    int32_t max_windows = 0;      // most windows of one output row
    int32_t* win_ptr = nullptr;   // [nlat_out + 1]
    DevWindow* windows = nullptr; // [nwin]
    float* vals = nullptr;        // [nnz, KP] float32, window order, zero padded
    // bf16 tap tables for the matrix-core fused kernel (see kernels_fused_mfma.hip)
    void* mfma_taps = nullptr;
    int64_t mfma_taps_bytes = 0;
    int32_t* mfma_row_info = nullptr;     // device copy of the info block
    std::vector<int32_t> mfma_info_host;  // host copy (offsets, tile options)
    int32_t mfma_ok = 0;
    // longitude-spectral tables for the spectral fused path (stride 1)
    void* spec_psih = nullptr;    // bf16 (re, im) words [nwin][K][spec_mp]
    int32_t spec_mp = 0;          // padded frequency count; 0 = no tables
    int32_t spec_radix[kSpecMaxRadix] = {0};
    int32_t spec_nrad = 0;
    std::vector<void*> allocations;
};

}  // namespace disco

struct disco_psi {
    disco::HostPsi host;
    disco::DevPsi dev;
};

namespace disco {

// Launchers (return DISCO_OK or DISCO_EHIP; arguments already validated).
int launch_contract(const disco_psi* psi, const void* x, int x_dtype, void* xk, int xk_dtype,
                    int B, int C, void* stream);
int launch_einsum(const void* xk, int xk_dtype, const void* w, int w_dtype, const float* bias,
                  void* y, int y_dtype, int B, int Ci, int Co, int groups, int K,
                  int nlat_out, int nlon_out, void* stream);
int launch_fused(const disco_psi* psi, const void* x, int dtype, const void* w,
                 const float* bias, void* y, int y_dtype, int B, int Ci, int Co, int groups,
                 void* stream);
// 1 if disco_fused_fwd takes the longitude-spectral path for these arguments
int fused_spectral_eligible(const disco_psi* psi, int x_dtype, int Ci, int Co, int groups);

// Scope around one kernel launch: while disco_kernel_timing(1) is in effect,
// records a HIP event on the launch stream at construction and at
// destruction, for disco_kernel_timing_read.  The name must be a string
// literal.
class KernelTimer {
  public:
    KernelTimer(const char* name, hipStream_t st);
    ~KernelTimer();
    KernelTimer(const KernelTimer&) = delete;
    KernelTimer& operator=(const KernelTimer&) = delete;

  private:
    const char* name_;
    hipStream_t st_;
    hipEvent_t start_ = nullptr, stop_ = nullptr;
    bool armed_ = false;
};

}  // namespace disco
