// Internal declarations shared by the host builder, the C-ABI layer and the
// HIP kernel launchers.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <functional>
#include <mutex>
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

// Runs fn(begin, end) over [0, n) in shares on up to 16 host threads.  A
// share whose thread cannot be started runs on the calling thread; an
// exception inside a share is caught.  Returns false if any share threw.
bool parallel_ranges(size_t n, const std::function<void(size_t, size_t)>& fn);

// Longitude-spectral tables (spectral_host.cpp), built for stride-1 layers
// whose longitude count N is even, at most kSpecMaxN, with N/2 a product of
// 2, 3 and 5, and K <= 8.  psih: [nwin][K][MP] bf16 (re, im) pairs in 32-bit
// words (real part low), Psi_hat of each window, followed by 32 zero words;
// radix: the plan of the N/2-point transform.  *mp = 0 when the layer
// does not qualify.
constexpr int kSpecMaxN = 1800;   // N/2 <= 900 bounds the transform butterflies per lane
constexpr int kSpecMaxRadix = 12;
int spectral_plan(int n, int32_t* radix, int32_t* nrad);
int build_spectral_tables(const HostPsi& h, std::vector<uint32_t>& psih, std::vector<float>& psih32,
                          int32_t* radix, int32_t* nrad, int32_t* mp);

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
    int32_t min_windows = 0;      // fewest windows of one output row
    int32_t t_max_windows = 0;    // most windows of one input row (transposed list)
    int32_t t_min_windows = 0;    // fewest windows of one input row
    int32_t* win_ptr = nullptr;   // [nlat_out + 1]
    DevWindow* windows = nullptr; // [nwin]
    float* vals = nullptr;        // [nnz, KP] float32, window order, zero padded
    // the same windows listed per input row (sorted by output row), for the
    // adjoint of the contraction; their `lat` field holds the output row
    int32_t* wint_ptr = nullptr;  // [nlat_in + 1]
    DevWindow* wins_t = nullptr;  // [nwin]
    // bf16 tap tables for the matrix-core fused kernel (see kernels_fused_mfma.hip)
    void* mfma_taps = nullptr;
    int64_t mfma_taps_bytes = 0;
    int32_t* mfma_row_info = nullptr;     // device copy of the info block
    std::vector<int32_t> mfma_info_host;  // host copy (offsets, tile options)
    int32_t mfma_ok = 0;
    // longitude-spectral tables for the spectral fused path (stride 1)
    void* spec_psih = nullptr;    // bf16 (re, im) words [nwin][K][spec_mp]
    float* spec_psih32 = nullptr; // float32 (re, im) pairs [nwin][K][spec_mp], or none
    void* spec_psih_t = nullptr;  // conj(Psi_hat) in the transposed window order (the adjoint)
    float* spec_psih32_t = nullptr;   // the same for the float32 table
    int32_t spec_mp = 0;          // padded frequency count; 0 = no tables
    int32_t spec_radix[kSpecMaxRadix] = {0};
    int32_t spec_nrad = 0;
    std::vector<void*> allocations;
};

// Device workspace that a Psi handle keeps between calls (the spectral
// algorithm's spectra, the matrix-core kernel's weight fragments).  It grows
// to the largest request and lives until the handle is freed.  `done` is
// recorded on the launch stream after every call that used it; a call on
// another stream first waits for it, so calls through one handle on several
// streams are ordered, not racing.
struct Workspace {
    std::mutex mu;
    void* ptr = nullptr;
    size_t cap = 0;
    hipEvent_t done = nullptr;
    hipStream_t last = nullptr;
    bool used = false;
};

}  // namespace disco

struct disco_psi {
    disco::HostPsi host;
    disco::DevPsi dev;
    mutable disco::Workspace ws;
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
// The fused forward on the direct algorithms only, with the weight fragments
// in the library's fixed device scratch (no allocation).
int launch_fused_noalloc(const disco_psi* psi, const void* x, int dtype, const void* w,
                         const float* bias, void* y, int y_dtype, int B, int Ci, int Co,
                         int groups, void* stream);
// The matrix-core contraction (kernels_fused_mfma.hip): bf16 x into a bf16
// [B, C, K, nlat_out, nlon_out] X_K, whole layer.  contract_mfma_ok says
// whether it takes these arguments; the launcher returns 0 when it does not
// (rc untouched), else 1 with *rc the result.
bool contract_mfma_ok(const disco_psi* psi, const void* x, const void* xk, int B, int C);
int try_launch_contract_mfma(const disco_psi* psi, const void* x, void* xk, int B, int C,
                             hipStream_t st, int* rc);
// 1 if disco_fused_fwd takes the longitude-spectral path for these arguments
int fused_spectral_eligible(const disco_psi* psi, int x_dtype, int Ci, int Co, int groups);
// The adjoint in x on the longitude-spectral kernels (stride-1 and stride-2
// layers with spectral tables, bf16 x, w and gy): 1 if it applies; the
// launcher returns 0 when it does not (rc untouched), else 1 with *rc the
// result.
int spectral_grad_x_eligible(const disco_psi* psi, int x_dtype, int gy_dtype, int Ci, int Co,
                             int groups);
int try_launch_grad_x_spectral(const disco_psi* psi, const void* gy, const void* w, void* gx,
                               int gx_dtype, int B, int Ci, int Co, hipStream_t st, int* rc);
// The same for float32 layers (stride 1, float32 x, w and gy), in float32.
int spectral_grad_x32_eligible(const disco_psi* psi, int Ci, int Co, int groups);
int try_launch_grad_x_spectral32(const disco_psi* psi, const void* gy, const void* w, void* gx,
                                 int gx_dtype, int B, int Ci, int Co, hipStream_t st, int* rc);

// Backward (kernels_backward.hip)
int launch_fill_zero(float* p, size_t n, void* stream);
int launch_contract_transpose(const disco_psi* psi, const void* gxk, int gxk_dtype, void* gx,
                              int gx_dtype, int B, int C, void* stream);
int launch_einsum_grad_xk(const void* gy, int gy_dtype, const void* w, int w_dtype, void* gxk,
                          int gxk_dtype, int B, int Ci, int Co, int groups, int K, int nlat_out,
                          int nlon_out, void* stream);
int launch_einsum_grad_w(const void* xk, int xk_dtype, const void* gy, int gy_dtype, float* gw,
                         int B, int Ci, int Co, int groups, int K, int nlat_out, int nlon_out,
                         void* stream);
int launch_fused_bwd(const disco_psi* psi, const void* x, int x_dtype, const void* w, int w_dtype,
                     const void* gy, int gy_dtype, void* gx, int gx_dtype, float* gw, float* gbias,
                     int B, int Ci, int Co, int groups, void* stream);

// Scope around one kernel launch: while disco_kernel_timing(1) is in effect,
// records a HIP event on the launch stream at construction and at
// destruction, for disco_kernel_timing_read.  The name must be a string
// literal.
// Scope around the launches of one call that use the handle's workspace:
// holds its lock, grows it to `bytes` (hipMalloc), orders the launch stream
// after the previous user's stream, and at destruction records `done` on the
// stream.  ptr() is null while the stream is being captured into a graph
// (the caller then allocates stream-ordered memory that the graph owns) and
// on failure (error() says which), and for a null handle.
class WorkspaceLease {
  public:
    WorkspaceLease(const disco_psi* psi, size_t bytes, hipStream_t st);
    ~WorkspaceLease();
    WorkspaceLease(const WorkspaceLease&) = delete;
    WorkspaceLease& operator=(const WorkspaceLease&) = delete;
    void* ptr() const { return ptr_; }
    int error() const { return rc_; }

  private:
    Workspace* ws_ = nullptr;
    hipStream_t st_ = nullptr;
    void* ptr_ = nullptr;
    int rc_ = DISCO_OK;
};
// Frees a handle's workspace (waits for its last user first).
void release_workspace(Workspace& ws);

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
