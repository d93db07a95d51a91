// C-ABI layer: argument checks, error reporting, handle lifetime and the
// device copy of Psi.  Compute entry points validate everything on the host
// before any launch and never fall back to another path.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>

#include "disco_internal.h"

namespace disco {

namespace {
thread_local std::string g_last_error;
}

int set_error(int code, const char* fmt, ...) {
    char buf[1024];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

void clear_error() { g_last_error.clear(); }

namespace {

int dtype_size(int dt) { return dt == DISCO_F32 ? 4 : (dt == DISCO_BF16 ? 2 : 0); }

bool valid_dtype(int dt) { return dt == DISCO_F32 || dt == DISCO_BF16; }

// A device pointer check: the pointer must be device (or managed) memory
// owned by the current device.
int check_device_ptr(const void* ptr, const char* name, int device) {
    if (ptr == nullptr) return set_error(DISCO_EINVAL, "%s is NULL", name);
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof(attr));
    hipError_t e = hipPointerGetAttributes(&attr, ptr);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return set_error(DISCO_EINVAL, "%s is not a device pointer known to HIP (%s)", name,
                         hipGetErrorString(e));
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
        return set_error(DISCO_EINVAL, "%s is not device memory", name);
    if (attr.device != device)
        return set_error(DISCO_EINVAL, "%s lives on device %d, the current device is %d", name,
                         attr.device, device);
    return DISCO_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const char* pa = static_cast<const char*>(a);
    const char* pb = static_cast<const char*>(b);
    return pa < pb + nb && pb < pa + na;
}

int current_device(int* dev) {
    hipError_t e = hipGetDevice(dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return set_error(DISCO_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    }
    return DISCO_OK;
}

int check_psi_on_device(const disco_psi* psi, int dev) {
    if (psi == nullptr) return set_error(DISCO_EINVAL, "psi handle is NULL");
    if (psi->dev.device < 0)
        return set_error(DISCO_EINVAL, "psi has no device copy: call disco_psi_to_device first");
    if (psi->dev.device != dev)
        return set_error(DISCO_EINVAL, "psi lives on device %d, the current device is %d",
                         psi->dev.device, dev);
    return DISCO_OK;
}

void free_device(disco::DevPsi& d) {
    for (void* p : d.allocations) (void)hipFree(p);
    d = disco::DevPsi();
}

}  // namespace

WorkspaceLease::WorkspaceLease(const disco_psi* psi, size_t bytes, hipStream_t st) : st_(st) {
    if (psi == nullptr) return;   // no lease wanted
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return;   // unknown: the caller allocates stream-ordered memory
    }
    if (cs != hipStreamCaptureStatusNone) return;
    Workspace& ws = psi->ws;
    ws.mu.lock();
    ws_ = &ws;
    if (bytes == 0) bytes = 256;
    if (ws.done == nullptr && hipEventCreateWithFlags(&ws.done, hipEventDisableTiming) != hipSuccess) {
        (void)hipGetLastError();
        ws.done = nullptr;
        rc_ = set_error(DISCO_EHIP, "hipEventCreateWithFlags for the workspace failed");
        return;
    }
    if (ws.cap < bytes) {
        if (ws.ptr != nullptr) {
            // the previous user may still run: wait, then free
            if (ws.used) (void)hipEventSynchronize(ws.done);
            (void)hipFree(ws.ptr);
            ws.ptr = nullptr;
            ws.cap = 0;
            ws.used = false;
        }
        hipError_t e = hipMalloc(&ws.ptr, bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            ws.ptr = nullptr;
            rc_ = set_error(e == hipErrorOutOfMemory ? DISCO_ENOMEM : DISCO_EHIP,
                            "hipMalloc(%zu) for the workspace failed: %s", bytes,
                            hipGetErrorString(e));
            return;
        }
        ws.cap = bytes;
    }
    if (ws.used && ws.last != st) {
        if (hipStreamWaitEvent(st, ws.done, 0) != hipSuccess) {
            (void)hipGetLastError();
            rc_ = set_error(DISCO_EHIP, "hipStreamWaitEvent on the workspace failed");
            return;
        }
    }
    ptr_ = ws.ptr;
}

WorkspaceLease::~WorkspaceLease() {
    if (ws_ == nullptr) return;
    if (ptr_ != nullptr) {
        if (hipEventRecord(ws_->done, st_) == hipSuccess) {
            ws_->last = st_;
            ws_->used = true;
        } else {
            // no event to order the next user by: make sure this use is over
            (void)hipGetLastError();
            (void)hipStreamSynchronize(st_);
            ws_->used = false;
        }
    }
    ws_->mu.unlock();
}

void release_workspace(Workspace& ws) {
    std::lock_guard<std::mutex> lock(ws.mu);
    if (ws.ptr != nullptr) {
        if (ws.used && ws.done != nullptr) (void)hipEventSynchronize(ws.done);
        (void)hipFree(ws.ptr);
    }
    if (ws.done != nullptr) (void)hipEventDestroy(ws.done);
    ws.ptr = nullptr;
    ws.cap = 0;
    ws.done = nullptr;
    ws.last = nullptr;
    ws.used = false;
}

namespace {

int dev_alloc(disco::DevPsi& d, void** ptr, size_t bytes) {
    if (bytes == 0) bytes = 16;
    hipError_t e = hipMalloc(ptr, bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return set_error(e == hipErrorOutOfMemory ? DISCO_ENOMEM : DISCO_EHIP,
                         "hipMalloc(%zu) failed: %s", bytes, hipGetErrorString(e));
    }
    d.allocations.push_back(*ptr);
    return DISCO_OK;
}

int dev_copy(void* dst, const void* src, size_t bytes) {
    if (bytes == 0) return DISCO_OK;
    hipError_t e = hipMemcpy(dst, src, bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return set_error(DISCO_EHIP, "hipMemcpy failed: %s", hipGetErrorString(e));
    }
    return DISCO_OK;
}

}  // namespace

int build_mfma_tables(disco_psi* psi, std::vector<char>& taps, std::vector<int32_t>& info);

}  // namespace disco

using namespace disco;

extern "C" {

const char* disco_version(void) { return "disco-gfx950 0.1.0"; }

const char* disco_last_error(void) { return g_last_error.c_str(); }

int disco_psi_build(const disco_psi_desc* desc, disco_psi** out) {
    clear_error();
    if (desc == nullptr || out == nullptr)
        return set_error(DISCO_EINVAL, "desc and out must not be NULL");
    *out = nullptr;
    disco_psi* psi = new (std::nothrow) disco_psi();
    if (psi == nullptr) return set_error(DISCO_ENOMEM, "host allocation failed");
    int rc = build_host_psi(*desc, psi->host);
    if (rc != DISCO_OK) {
        delete psi;
        return rc;
    }
    *out = psi;
    return DISCO_OK;
}

int disco_psi_query(const disco_psi* psi, int32_t* K, int64_t* nnz, int64_t* nnz_nonzero,
                    double* theta_cutoff) {
    clear_error();
    if (psi == nullptr) return set_error(DISCO_EINVAL, "psi handle is NULL");
    if (K) *K = psi->host.K;
    if (nnz) *nnz = (int64_t)psi->host.in_lat.size();
    if (nnz_nonzero) *nnz_nonzero = psi->host.nnz_nonzero;
    if (theta_cutoff) *theta_cutoff = psi->host.cutoff;
    return DISCO_OK;
}

int disco_psi_export(const disco_psi* psi, int64_t* row_ptr, int32_t* in_lat, int32_t* lon_off,
                     double* vals) {
    clear_error();
    if (psi == nullptr) return set_error(DISCO_EINVAL, "psi handle is NULL");
    const HostPsi& h = psi->host;
    if (row_ptr) std::memcpy(row_ptr, h.row_ptr.data(), h.row_ptr.size() * sizeof(int64_t));
    if (in_lat) std::memcpy(in_lat, h.in_lat.data(), h.in_lat.size() * sizeof(int32_t));
    if (lon_off) std::memcpy(lon_off, h.lon_off.data(), h.lon_off.size() * sizeof(int32_t));
    if (vals) std::memcpy(vals, h.vals.data(), h.vals.size() * sizeof(double));
    return DISCO_OK;
}

int disco_psi_to_device(disco_psi* psi) {
    clear_error();
    if (psi == nullptr) return set_error(DISCO_EINVAL, "psi handle is NULL");
    int dev = -1;
    int rc = current_device(&dev);
    if (rc != DISCO_OK) return rc;
    if (psi->dev.device == dev) return DISCO_OK;
    if (psi->dev.device >= 0)
        return set_error(DISCO_EINVAL, "psi already lives on device %d (current device %d)",
                         psi->dev.device, dev);
    const HostPsi& h = psi->host;
    DevPsi d;
    const int K = h.K;
    int KP = 1;
    while (KP < K) KP *= 2;
    if (KP > 8) KP = (K + 3) / 4 * 4;
    d.KP = KP;
    const int nlat_out = h.desc.nlat_out;
    std::vector<int32_t> wptr(nlat_out + 1);
    std::vector<DevWindow> wins(h.windows.size());
    const int64_t npts = (int64_t)(h.win_vals.size() / K);
    std::vector<float> vals;
    try {
        vals.assign((size_t)npts * KP, 0.0f);
    } catch (const std::bad_alloc&) {
        return set_error(DISCO_ENOMEM, "host allocation failed");
    }
    for (int64_t p = 0; p < npts; ++p)
        for (int k = 0; k < K; ++k) vals[p * KP + k] = (float)h.win_vals[p * K + k];
    for (int j = 0; j <= nlat_out; ++j) wptr[j] = (int32_t)h.win_ptr[j];
    for (size_t n = 0; n < h.windows.size(); ++n) {
        wins[n].lat = h.windows[n].lat;
        wins[n].p_lo = h.windows[n].p_lo;
        wins[n].width = h.windows[n].width;
        wins[n].val_off = (int32_t)h.windows[n].val_off;
        d.max_width = std::max(d.max_width, h.windows[n].width);
    }
    // the transposed list: windows grouped by input row, then by output row
    const int nlat_in = h.desc.nlat_in;
    std::vector<int32_t> wtptr(nlat_in + 1, 0);
    std::vector<DevWindow> wins_t(wins.size());
    std::vector<int32_t> orig_t(wins.size());   // forward index of each transposed window
    {
        std::vector<int32_t> out_row(wins.size());
        for (int j = 0; j < nlat_out; ++j)
            for (int n = wptr[j]; n < wptr[j + 1]; ++n) out_row[n] = j;
        for (const DevWindow& w : wins) ++wtptr[w.lat + 1];
        for (int i = 0; i < nlat_in; ++i) wtptr[i + 1] += wtptr[i];
        std::vector<int32_t> fill(wtptr.begin(), wtptr.end() - 1);
        // forward windows are in output-row order, so each input row's list
        // comes out sorted by output row
        for (size_t n = 0; n < wins.size(); ++n) {
            DevWindow t = wins[n];
            t.lat = out_row[n];
            orig_t[fill[wins[n].lat]] = (int32_t)n;
            wins_t[fill[wins[n].lat]++] = t;
        }
    }
    d.min_windows = nlat_out > 0 ? wptr[1] - wptr[0] : 0;
    d.t_min_windows = nlat_in > 0 ? wtptr[1] - wtptr[0] : 0;
    for (int i = 0; i < nlat_in; ++i) {
        d.t_max_windows = std::max(d.t_max_windows, wtptr[i + 1] - wtptr[i]);
        d.t_min_windows = std::min(d.t_min_windows, wtptr[i + 1] - wtptr[i]);
    }
    for (int j = 0; j < nlat_out; ++j) {
        d.max_windows = std::max(d.max_windows, wptr[j + 1] - wptr[j]);
        d.min_windows = std::min(d.min_windows, wptr[j + 1] - wptr[j]);
        d.max_row_points = std::max(
            d.max_row_points, (int32_t)(h.row_ptr[j + 1] - h.row_ptr[j]));
    }
    std::vector<char> taps;
    std::vector<int32_t> info;
    rc = build_mfma_tables(psi, taps, info);
    if (rc != DISCO_OK) return rc;
    std::vector<uint32_t> spec_psih;
    std::vector<float> spec_psih32;
    rc = build_spectral_tables(h, spec_psih, spec_psih32, d.spec_radix, &d.spec_nrad, &d.spec_mp);
    if (rc != DISCO_OK) return rc;

    void* p = nullptr;
    if ((rc = dev_alloc(d, &p, wptr.size() * sizeof(int32_t))) != DISCO_OK) goto fail;
    d.win_ptr = static_cast<int32_t*>(p);
    if ((rc = dev_copy(p, wptr.data(), wptr.size() * sizeof(int32_t))) != DISCO_OK) goto fail;
    if ((rc = dev_alloc(d, &p, wins.size() * sizeof(DevWindow))) != DISCO_OK) goto fail;
    d.windows = static_cast<DevWindow*>(p);
    if ((rc = dev_copy(p, wins.data(), wins.size() * sizeof(DevWindow))) != DISCO_OK) goto fail;
    if ((rc = dev_alloc(d, &p, wtptr.size() * sizeof(int32_t))) != DISCO_OK) goto fail;
    d.wint_ptr = static_cast<int32_t*>(p);
    if ((rc = dev_copy(p, wtptr.data(), wtptr.size() * sizeof(int32_t))) != DISCO_OK) goto fail;
    if ((rc = dev_alloc(d, &p, wins_t.size() * sizeof(DevWindow))) != DISCO_OK) goto fail;
    d.wins_t = static_cast<DevWindow*>(p);
    if ((rc = dev_copy(p, wins_t.data(), wins_t.size() * sizeof(DevWindow))) != DISCO_OK) goto fail;
    if ((rc = dev_alloc(d, &p, vals.size() * sizeof(float))) != DISCO_OK) goto fail;
    d.vals = static_cast<float*>(p);
    if ((rc = dev_copy(p, vals.data(), vals.size() * sizeof(float))) != DISCO_OK) goto fail;
    if (!taps.empty()) {
        if ((rc = dev_alloc(d, &p, taps.size())) != DISCO_OK) goto fail;
        d.mfma_taps = p;
        d.mfma_taps_bytes = (int64_t)taps.size();
        if ((rc = dev_copy(p, taps.data(), taps.size())) != DISCO_OK) goto fail;
        if ((rc = dev_alloc(d, &p, info.size() * sizeof(int32_t))) != DISCO_OK) goto fail;
        d.mfma_row_info = static_cast<int32_t*>(p);
        if ((rc = dev_copy(p, info.data(), info.size() * sizeof(int32_t))) != DISCO_OK) goto fail;
        d.mfma_info_host = info;
        d.mfma_ok = 1;
    }
    if (d.spec_mp > 0) {
        if ((rc = dev_alloc(d, &p, spec_psih.size() * sizeof(uint32_t))) != DISCO_OK) goto fail;
        d.spec_psih = p;
        if ((rc = dev_copy(p, spec_psih.data(), spec_psih.size() * sizeof(uint32_t))) != DISCO_OK)
            goto fail;
        if (h.stride == 1 || h.stride == 2) {
            // the adjoint's table: windows in the transposed order, each
            // Psi_hat conjugated (the matrix-core kernel multiplies by the
            // conjugate of its table, and the adjoint of the correlation is
            // the convolution, Psi_hat itself); the same trailing zero block
            const size_t blk = (size_t)h.K * d.spec_mp;
            std::vector<uint32_t> pt;
            try {
                pt.assign(spec_psih.size(), 0u);
            } catch (const std::bad_alloc&) {
                rc = set_error(DISCO_ENOMEM, "host allocation for the adjoint table failed");
                goto fail;
            }
            for (size_t n = 0; n < wins_t.size(); ++n) {
                const uint32_t* src = spec_psih.data() + (size_t)orig_t[n] * blk;
                uint32_t* dst = pt.data() + n * blk;
                for (size_t e = 0; e < blk; ++e) dst[e] = src[e] ^ 0x80000000u;   // imag sign
            }
            if ((rc = dev_alloc(d, &p, pt.size() * sizeof(uint32_t))) != DISCO_OK) goto fail;
            d.spec_psih_t = p;
            if ((rc = dev_copy(p, pt.data(), pt.size() * sizeof(uint32_t))) != DISCO_OK) goto fail;
        }
        if (!spec_psih32.empty() && h.stride == 1) {
            // the float32 adjoint's table: transposed order, imaginary parts negated
            const size_t blk = (size_t)h.K * d.spec_mp * 2;
            std::vector<float> pt;
            try {
                pt.assign(spec_psih32.size(), 0.0f);
            } catch (const std::bad_alloc&) {
                rc = set_error(DISCO_ENOMEM, "host allocation for the adjoint table failed");
                goto fail;
            }
            for (size_t n = 0; n < wins_t.size(); ++n) {
                const float* src = spec_psih32.data() + (size_t)orig_t[n] * blk;
                float* dst = pt.data() + n * blk;
                for (size_t e = 0; e < blk; e += 2) {
                    dst[e] = src[e];
                    dst[e + 1] = -src[e + 1];
                }
            }
            if ((rc = dev_alloc(d, &p, pt.size() * sizeof(float))) != DISCO_OK) goto fail;
            d.spec_psih32_t = static_cast<float*>(p);
            if ((rc = dev_copy(p, pt.data(), pt.size() * sizeof(float))) != DISCO_OK) goto fail;
        }
        if (!spec_psih32.empty()) {
            if ((rc = dev_alloc(d, &p, spec_psih32.size() * sizeof(float))) != DISCO_OK) goto fail;
            d.spec_psih32 = static_cast<float*>(p);
            if ((rc = dev_copy(p, spec_psih32.data(), spec_psih32.size() * sizeof(float))) !=
                DISCO_OK)
                goto fail;
        }
    }
    d.device = dev;
    psi->dev = d;
    return DISCO_OK;
fail:
    free_device(d);
    return rc;
}

void disco_psi_free(disco_psi* psi) {
    if (psi == nullptr) return;
    if (psi->dev.device >= 0) {
        int cur = -1;
        if (hipGetDevice(&cur) == hipSuccess && cur != psi->dev.device) {
            (void)hipSetDevice(psi->dev.device);
            release_workspace(psi->ws);
            free_device(psi->dev);
            (void)hipSetDevice(cur);
        } else {
            release_workspace(psi->ws);
            free_device(psi->dev);
        }
    }
    delete psi;
}

int disco_contract(const disco_psi* psi, const void* x, int x_dtype, void* xk, int xk_dtype,
                   int32_t B, int32_t C, void* stream) {
    clear_error();
    if (psi == nullptr) return set_error(DISCO_EINVAL, "psi handle is NULL");
    if (!valid_dtype(x_dtype) || !valid_dtype(xk_dtype))
        return set_error(DISCO_EINVAL, "unknown dtype code (x %d, xk %d)", x_dtype, xk_dtype);
    if (B < 0 || C < 0) return set_error(DISCO_EINVAL, "B and C must be >= 0 (got %d, %d)", B, C);
    if (B == 0 || C == 0) return DISCO_OK;
    int dev = -1;
    int rc = current_device(&dev);
    if (rc != DISCO_OK) return rc;
    if ((rc = check_psi_on_device(psi, dev)) != DISCO_OK) return rc;
    if ((rc = check_device_ptr(x, "x", dev)) != DISCO_OK) return rc;
    if ((rc = check_device_ptr(xk, "xk", dev)) != DISCO_OK) return rc;
    const disco_psi_desc& d = psi->host.desc;
    const size_t nx = (size_t)B * C * d.nlat_in * d.nlon_in * dtype_size(x_dtype);
    const size_t nxk = (size_t)B * C * psi->host.K * d.nlat_out * d.nlon_out * dtype_size(xk_dtype);
    if (overlap(x, nx, xk, nxk)) return set_error(DISCO_EINVAL, "x and xk overlap");
    return launch_contract(psi, x, x_dtype, xk, xk_dtype, B, C, stream);
}

int disco_einsum(const void* xk, int xk_dtype, const void* w, int w_dtype, const float* bias,
                 void* y, int y_dtype, int32_t B, int32_t Ci, int32_t Co, int32_t groups,
                 int32_t K, int32_t nlat_out, int32_t nlon_out, void* stream) {
    clear_error();
    if (!valid_dtype(xk_dtype) || !valid_dtype(w_dtype) || !valid_dtype(y_dtype))
        return set_error(DISCO_EINVAL, "unknown dtype code (xk %d, w %d, y %d)", xk_dtype,
                         w_dtype, y_dtype);
    if (xk_dtype != w_dtype)
        return set_error(DISCO_EUNSUPPORTED, "xk and w must have the same dtype");
    if (B < 0 || Ci < 1 || Co < 1 || K < 1 || nlat_out < 1 || nlon_out < 1)
        return set_error(DISCO_EINVAL, "sizes must be positive (B %d Ci %d Co %d K %d nlat_out %d "
                         "nlon_out %d)", B, Ci, Co, K, nlat_out, nlon_out);
    if (groups < 1 || Ci % groups != 0 || Co % groups != 0)
        return set_error(DISCO_EINVAL,
                         "groups (%d) must divide in_channels (%d) and out_channels (%d)", groups,
                         Ci, Co);
    if (B == 0) return DISCO_OK;
    int dev = -1;
    int rc = current_device(&dev);
    if (rc != DISCO_OK) return rc;
    if ((rc = check_device_ptr(xk, "xk", dev)) != DISCO_OK) return rc;
    if ((rc = check_device_ptr(w, "w", dev)) != DISCO_OK) return rc;
    if ((rc = check_device_ptr(y, "y", dev)) != DISCO_OK) return rc;
    if (bias && (rc = check_device_ptr(bias, "bias", dev)) != DISCO_OK) return rc;
    const size_t hw = (size_t)nlat_out * nlon_out;
    const size_t nxk = (size_t)B * Ci * K * hw * dtype_size(xk_dtype);
    const size_t nw = (size_t)Co * (Ci / groups) * K * dtype_size(w_dtype);
    const size_t ny = (size_t)B * Co * hw * dtype_size(y_dtype);
    if (overlap(y, ny, xk, nxk) || overlap(y, ny, w, nw) || (bias && overlap(y, ny, bias, Co * 4)))
        return set_error(DISCO_EINVAL, "y overlaps an input");
    return launch_einsum(xk, xk_dtype, w, w_dtype, bias, y, y_dtype, B, Ci, Co, groups, K,
                         nlat_out, nlon_out, stream);
}

int disco_fused_is_spectral(const disco_psi* psi, int x_dtype, int32_t Ci, int32_t Co,
                            int32_t groups) {
    clear_error();
    if (psi == nullptr) return set_error(DISCO_EINVAL, "psi handle is NULL");
    if (psi->dev.device < 0) return set_error(DISCO_EINVAL, "psi is not on a device");
    return fused_spectral_eligible(psi, x_dtype, Ci, Co, groups);
}

}  // extern "C"

namespace {
// Argument checks shared by the two fused entry points; *skip = true for an
// empty batch (nothing to do).
int check_fused_args(const disco_psi* psi, const void* x, int x_dtype, const void* w, int w_dtype,
                     const float* bias, void* y, int y_dtype, int32_t B, int32_t Ci, int32_t Co,
                     int32_t groups, bool* skip) {
    *skip = false;
    if (psi == nullptr) return set_error(DISCO_EINVAL, "psi handle is NULL");
    if (!valid_dtype(x_dtype) || !valid_dtype(w_dtype) || !valid_dtype(y_dtype))
        return set_error(DISCO_EINVAL, "unknown dtype code (x %d, w %d, y %d)", x_dtype, w_dtype,
                         y_dtype);
    if (x_dtype != w_dtype)
        return set_error(DISCO_EUNSUPPORTED, "x and w must have the same dtype");
    if (B < 0 || Ci < 1 || Co < 1)
        return set_error(DISCO_EINVAL, "sizes must be positive (B %d Ci %d Co %d)", B, Ci, Co);
    if (groups < 1 || Ci % groups != 0 || Co % groups != 0)
        return set_error(DISCO_EINVAL,
                         "groups (%d) must divide in_channels (%d) and out_channels (%d)", groups,
                         Ci, Co);
    if (B == 0) {
        *skip = true;
        return DISCO_OK;
    }
    int dev = -1;
    int rc = current_device(&dev);
    if (rc != DISCO_OK) return rc;
    if ((rc = check_psi_on_device(psi, dev)) != DISCO_OK) return rc;
    if ((rc = check_device_ptr(x, "x", dev)) != DISCO_OK) return rc;
    if ((rc = check_device_ptr(w, "w", dev)) != DISCO_OK) return rc;
    if ((rc = check_device_ptr(y, "y", dev)) != DISCO_OK) return rc;
    if (bias && (rc = check_device_ptr(bias, "bias", dev)) != DISCO_OK) return rc;
    const disco_psi_desc& d = psi->host.desc;
    const size_t nx = (size_t)B * Ci * d.nlat_in * d.nlon_in * dtype_size(x_dtype);
    const size_t nw = (size_t)Co * (Ci / groups) * psi->host.K * dtype_size(w_dtype);
    const size_t ny = (size_t)B * Co * d.nlat_out * d.nlon_out * dtype_size(y_dtype);
    if (overlap(y, ny, x, nx) || overlap(y, ny, w, nw) || (bias && overlap(y, ny, bias, Co * 4)))
        return set_error(DISCO_EINVAL, "y overlaps an input");
    return DISCO_OK;
}
}  // namespace

extern "C" {

int disco_fused_fwd(const disco_psi* psi, const void* x, int x_dtype, const void* w, int w_dtype,
                    const float* bias, void* y, int y_dtype, int32_t B, int32_t Ci, int32_t Co,
                    int32_t groups, void* stream) {
    clear_error();
    bool skip = false;
    int rc = check_fused_args(psi, x, x_dtype, w, w_dtype, bias, y, y_dtype, B, Ci, Co, groups,
                              &skip);
    if (rc != DISCO_OK || skip) return rc;
    return launch_fused(psi, x, x_dtype, w, bias, y, y_dtype, B, Ci, Co, groups, stream);
}

int disco_fused_fwd_noalloc(const disco_psi* psi, const void* x, int x_dtype, const void* w,
                            int w_dtype, const float* bias, void* y, int y_dtype, int32_t B,
                            int32_t Ci, int32_t Co, int32_t groups, void* stream) {
    clear_error();
    bool skip = false;
    int rc = check_fused_args(psi, x, x_dtype, w, w_dtype, bias, y, y_dtype, B, Ci, Co, groups,
                              &skip);
    if (rc != DISCO_OK || skip) return rc;
    return launch_fused_noalloc(psi, x, x_dtype, w, bias, y, y_dtype, B, Ci, Co, groups, stream);
}

int disco_contract_transpose(const disco_psi* psi, const void* gxk, int gxk_dtype, void* gx,
                             int gx_dtype, int32_t B, int32_t C, void* stream) {
    clear_error();
    if (psi == nullptr) return set_error(DISCO_EINVAL, "psi handle is NULL");
    if (!valid_dtype(gxk_dtype) || !valid_dtype(gx_dtype))
        return set_error(DISCO_EINVAL, "unknown dtype code (gxk %d, gx %d)", gxk_dtype, gx_dtype);
    if (B < 0 || C < 0) return set_error(DISCO_EINVAL, "B and C must be >= 0 (got %d, %d)", B, C);
    if (B == 0 || C == 0) return DISCO_OK;
    int dev = -1;
    int rc = current_device(&dev);
    if (rc != DISCO_OK) return rc;
    if ((rc = check_psi_on_device(psi, dev)) != DISCO_OK) return rc;
    if ((rc = check_device_ptr(gxk, "gxk", dev)) != DISCO_OK) return rc;
    if ((rc = check_device_ptr(gx, "gx", dev)) != DISCO_OK) return rc;
    const disco_psi_desc& d = psi->host.desc;
    const size_t ngx = (size_t)B * C * d.nlat_in * d.nlon_in * dtype_size(gx_dtype);
    const size_t ngxk =
        (size_t)B * C * psi->host.K * d.nlat_out * d.nlon_out * dtype_size(gxk_dtype);
    if (overlap(gx, ngx, gxk, ngxk)) return set_error(DISCO_EINVAL, "gx and gxk overlap");
    return launch_contract_transpose(psi, gxk, gxk_dtype, gx, gx_dtype, B, C, stream);
}

namespace {
int check_einsum_sizes(int32_t B, int32_t Ci, int32_t Co, int32_t groups, int32_t K,
                       int32_t nlat_out, int32_t nlon_out) {
    if (B < 0 || Ci < 1 || Co < 1 || K < 1 || nlat_out < 1 || nlon_out < 1)
        return set_error(DISCO_EINVAL, "sizes must be positive (B %d Ci %d Co %d K %d nlat_out %d "
                         "nlon_out %d)", B, Ci, Co, K, nlat_out, nlon_out);
    if (groups < 1 || Ci % groups != 0 || Co % groups != 0)
        return set_error(DISCO_EINVAL,
                         "groups (%d) must divide in_channels (%d) and out_channels (%d)", groups,
                         Ci, Co);
    return DISCO_OK;
}
}  // namespace

int disco_einsum_grad_xk(const void* gy, int gy_dtype, const void* w, int w_dtype, void* gxk,
                         int gxk_dtype, int32_t B, int32_t Ci, int32_t Co, int32_t groups,
                         int32_t K, int32_t nlat_out, int32_t nlon_out, void* stream) {
    clear_error();
    if (!valid_dtype(gy_dtype) || !valid_dtype(w_dtype) || !valid_dtype(gxk_dtype))
        return set_error(DISCO_EINVAL, "unknown dtype code (gy %d, w %d, gxk %d)", gy_dtype,
                         w_dtype, gxk_dtype);
    int rc = check_einsum_sizes(B, Ci, Co, groups, K, nlat_out, nlon_out);
    if (rc != DISCO_OK || B == 0) return rc;
    int dev = -1;
    if ((rc = current_device(&dev)) != DISCO_OK) return rc;
    if ((rc = check_device_ptr(gy, "gy", dev)) != DISCO_OK) return rc;
    if ((rc = check_device_ptr(w, "w", dev)) != DISCO_OK) return rc;
    if ((rc = check_device_ptr(gxk, "gxk", dev)) != DISCO_OK) return rc;
    const size_t hw = (size_t)nlat_out * nlon_out;
    const size_t ngxk = (size_t)B * Ci * K * hw * dtype_size(gxk_dtype);
    const size_t ngy = (size_t)B * Co * hw * dtype_size(gy_dtype);
    const size_t nw = (size_t)Co * (Ci / groups) * K * dtype_size(w_dtype);
    if (overlap(gxk, ngxk, gy, ngy) || overlap(gxk, ngxk, w, nw))
        return set_error(DISCO_EINVAL, "gxk overlaps an input");
    return launch_einsum_grad_xk(gy, gy_dtype, w, w_dtype, gxk, gxk_dtype, B, Ci, Co, groups, K,
                                 nlat_out, nlon_out, stream);
}

int disco_einsum_grad_w(const void* xk, int xk_dtype, const void* gy, int gy_dtype, float* gw,
                        int32_t B, int32_t Ci, int32_t Co, int32_t groups, int32_t K,
                        int32_t nlat_out, int32_t nlon_out, void* stream) {
    clear_error();
    if (!valid_dtype(xk_dtype) || !valid_dtype(gy_dtype))
        return set_error(DISCO_EINVAL, "unknown dtype code (xk %d, gy %d)", xk_dtype, gy_dtype);
    int rc = check_einsum_sizes(B, Ci, Co, groups, K, nlat_out, nlon_out);
    if (rc != DISCO_OK) return rc;
    int dev = -1;
    if ((rc = current_device(&dev)) != DISCO_OK) return rc;
    if ((rc = check_device_ptr(gw, "gw", dev)) != DISCO_OK) return rc;
    const size_t ngw = (size_t)Co * (Ci / groups) * K;
    if (B == 0) return launch_fill_zero(gw, ngw, stream);   // an empty sum
    if ((rc = check_device_ptr(xk, "xk", dev)) != DISCO_OK) return rc;
    if ((rc = check_device_ptr(gy, "gy", dev)) != DISCO_OK) return rc;
    const size_t hw = (size_t)nlat_out * nlon_out;
    const size_t nxk = (size_t)B * Ci * K * hw * dtype_size(xk_dtype);
    const size_t ngy = (size_t)B * Co * hw * dtype_size(gy_dtype);
    if (overlap(gw, ngw * 4, xk, nxk) || overlap(gw, ngw * 4, gy, ngy))
        return set_error(DISCO_EINVAL, "gw overlaps an input");
    return launch_einsum_grad_w(xk, xk_dtype, gy, gy_dtype, gw, B, Ci, Co, groups, K, nlat_out,
                                nlon_out, stream);
}

int disco_fused_bwd(const disco_psi* psi, const void* x, int x_dtype, const void* w, int w_dtype,
                    const void* gy, int gy_dtype, void* gx, int gx_dtype, float* gw, float* gbias,
                    int32_t B, int32_t Ci, int32_t Co, int32_t groups, void* stream) {
    clear_error();
    if (psi == nullptr) return set_error(DISCO_EINVAL, "psi handle is NULL");
    if (!valid_dtype(x_dtype) || !valid_dtype(w_dtype) || !valid_dtype(gy_dtype) ||
        (gx && !valid_dtype(gx_dtype)))
        return set_error(DISCO_EINVAL, "unknown dtype code (x %d, w %d, gy %d, gx %d)", x_dtype,
                         w_dtype, gy_dtype, gx_dtype);
    if (gx == nullptr && gw == nullptr && gbias == nullptr)
        return set_error(DISCO_EINVAL, "gx, gw and gbias are all NULL: nothing to compute");
    const disco_psi_desc& d = psi->host.desc;
    const int K = psi->host.K;
    int rc = check_einsum_sizes(B, Ci, Co, groups, K, d.nlat_out, d.nlon_out);
    if (rc != DISCO_OK) return rc;
    int dev = -1;
    if ((rc = current_device(&dev)) != DISCO_OK) return rc;
    if ((rc = check_psi_on_device(psi, dev)) != DISCO_OK) return rc;
    if (gw && (rc = check_device_ptr(gw, "gw", dev)) != DISCO_OK) return rc;
    if (gbias && (rc = check_device_ptr(gbias, "gbias", dev)) != DISCO_OK) return rc;
    const size_t ngw = (size_t)Co * (Ci / groups) * K;
    if (B == 0) {   // empty sums; gx has no elements
        if (gw && (rc = launch_fill_zero(gw, ngw, stream)) != DISCO_OK) return rc;
        if (gbias && (rc = launch_fill_zero(gbias, (size_t)Co, stream)) != DISCO_OK) return rc;
        return DISCO_OK;
    }
    if ((rc = check_device_ptr(gy, "gy", dev)) != DISCO_OK) return rc;
    if ((gx || gw) && (rc = check_device_ptr(x, "x", dev)) != DISCO_OK) return rc;
    if (gx && (rc = check_device_ptr(w, "w", dev)) != DISCO_OK) return rc;
    if (gx && (rc = check_device_ptr(gx, "gx", dev)) != DISCO_OK) return rc;
    const size_t nx = (size_t)B * Ci * d.nlat_in * d.nlon_in * dtype_size(x_dtype);
    const size_t nw = (size_t)Co * (Ci / groups) * K * dtype_size(w_dtype);
    const size_t ngy = (size_t)B * Co * d.nlat_out * d.nlon_out * dtype_size(gy_dtype);
    const size_t ngx = gx ? (size_t)B * Ci * d.nlat_in * d.nlon_in * dtype_size(gx_dtype) : 0;
    struct Span {
        const void* p;
        size_t n;
    };
    const Span outs[3] = {{gx, ngx}, {gw, gw ? ngw * 4 : 0}, {gbias, gbias ? (size_t)Co * 4 : 0}};
    const Span ins[3] = {{x, (gx || gw) ? nx : 0}, {w, gx ? nw : 0}, {gy, ngy}};
    for (int a = 0; a < 3; ++a) {
        if (!outs[a].p) continue;
        for (int b2 = 0; b2 < 3; ++b2)
            if (ins[b2].p && overlap(outs[a].p, outs[a].n, ins[b2].p, ins[b2].n))
                return set_error(DISCO_EINVAL, "a gradient output overlaps an input");
        for (int b2 = a + 1; b2 < 3; ++b2)
            if (outs[b2].p && overlap(outs[a].p, outs[a].n, outs[b2].p, outs[b2].n))
                return set_error(DISCO_EINVAL, "gradient outputs overlap");
    }
    return launch_fused_bwd(psi, x, x_dtype, w, w_dtype, gy, gy_dtype, gx, gx_dtype, gw, gbias, B,
                            Ci, Co, groups, stream);
}

}  // extern "C"
