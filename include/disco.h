/*
 * disco.h - C ABI of the MI355X (gfx950) forward DISCO convolution on the 2-sphere.
 *
 * The operation (torch_harmonics.DiscreteContinuousConvS2 page, forward
 * equation and the paragraph defining Psi):
 *
 *   g[b,co,j,q] = sum_{ci,k} w[co,ci,k] * sum_{(i,p)} Psi[k,j,(i,p)] * x[b,ci,i,(q*s+p) mod nlon_in]
 *
 * with s = nlon_in / nlon_out.  Psi holds the piecewise-linear filter-basis
 * values at input points seen from the output point (theta'_j, 0) after it is
 * rotated to the north pole, times the quadrature weights; it does not depend
 * on the output longitude q (p-shift symmetry, same page).
 *
 * Conventions shared by every entry point
 *  - Tensors are caller-owned, dense, row-major (C order), and are never
 *    retained or freed by the library:
 *      x   [B, Ci, nlat_in, nlon_in]            (the layer input; page: forward())
 *      xk  [B, Ci, K, nlat_out, nlon_out]       (K-expanded intermediate; the
 *                                                DistributedDiscreteContinuousConvS2
 *                                                page, polar_mode parameter, names this shape)
 *      w   [Co, Ci/groups, K]
 *      y   [B, Co, nlat_out, nlon_out]          (the layer output)
 *      bias [Co] float32, or NULL for no bias.
 *  - Compute entry points take DEVICE pointers on the current HIP device and a
 *    hipStream_t passed as void* (NULL = default stream).  Work is enqueued on
 *    that stream and the call returns without waiting.  Every argument is
 *    checked before anything is launched; a failed check launches nothing.
 *  - Return value: DISCO_OK or a negative DISCO_E* code; disco_last_error()
 *    then gives a message for the calling thread.  The library never aborts
 *    and never falls back to another code path or to the CPU.
 *  - dtype codes: DISCO_F32 (float32) and DISCO_BF16 (bfloat16).  Products
 *    and sums are accumulated in float32.
 */
#ifndef DISCO_H
#define DISCO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define DISCO_OK             0
#define DISCO_EINVAL        -1   /* invalid argument (bad size, null pointer, non-divisible groups, ...) */
#define DISCO_EUNSUPPORTED  -2   /* valid request this library does not implement */
#define DISCO_ENOMEM        -3   /* host or device allocation failed */
#define DISCO_EHIP          -4   /* a HIP runtime call or kernel launch failed */

/* element types */
#define DISCO_F32   0
#define DISCO_BF16  1

/* grids (DiscreteContinuousConvS2 page, grid_in / grid_out parameters) */
/* Every grid is a rule in x = cos(theta) over [-1, 1] (weights sum to 2),
 * times 2*pi/nlon per point; nodes ordered from the north pole.  The pages
 * name the last three (DistributedSpectralConvS2 page, grid_in) without
 * defining them; these are the textbook rules of those names. */
#define DISCO_GRID_EQUIANGULAR 0  /* theta_i = pi*i/(nlat-1) (both poles), Clenshaw-Curtis weights */
#define DISCO_GRID_LEGENDRE_GAUSS 1  /* Gauss-Legendre nodes and weights (no poles) */
#define DISCO_GRID_LOBATTO 2      /* Gauss-Lobatto-Legendre nodes (both poles) and weights */
#define DISCO_GRID_EQUIANGULAR_TRAPEZOIDAL 3  /* equiangular nodes, composite trapezoid in x */

/* basis (same page, basis_type / basis_norm_mode parameters) */
#define DISCO_BASIS_PIECEWISE_LINEAR 0
#define DISCO_NORM_NONE 0         /* Psi = basis value * quadrature weight, no further scaling */

typedef struct disco_psi disco_psi;   /* opaque, library-owned, immutable after build */

/* Problem description (same page: in_shape, out_shape, kernel_shape,
 * basis_type, basis_norm_mode, grid_in, grid_out, theta_cutoff). */
typedef struct disco_psi_desc {
    int32_t nlat_in, nlon_in;       /* input grid */
    int32_t nlat_out, nlon_out;     /* output grid; nlon_in must be a multiple of nlon_out */
    int32_t grid_in, grid_out;      /* DISCO_GRID_* */
    int32_t basis_type;             /* DISCO_BASIS_PIECEWISE_LINEAR */
    int32_t basis_norm;             /* DISCO_NORM_NONE */
    int32_t kernel_shape[2];        /* {nr, nphi}: nphi = 0 -> isotropic (nr,), K = nr;
                                       nphi >= 1 -> K = 1 + (nr-1)*nphi */
    double  theta_cutoff;           /* radians, in (0, pi); <= 0 selects (nr+1)*pi/(nlat_out-1) */
} disco_psi_desc;

/* Build Psi on the host in float64 (DiscreteContinuousConvS2 page, Psi
 * paragraph).  No GPU is touched.  On success *out owns a new handle; free it
 * with disco_psi_free.  EINVAL for inconsistent sizes or cutoff, EUNSUPPORTED
 * for unknown grid codes, other bases/normalisations or K > 64, ENOMEM on
 * allocation failure. */
int disco_psi_build(const disco_psi_desc* desc, disco_psi** out);

/* Sizes of a built Psi: number of basis functions K, support points nnz (the
 * (j,i,p) triples with r < theta_cutoff), entries with a basis value above
 * 1e-12 before weighting, and the cutoff actually used.  Any output pointer
 * may be NULL. */
int disco_psi_query(const disco_psi* psi, int32_t* K, int64_t* nnz,
                    int64_t* nnz_nonzero, double* theta_cutoff);

/* Copy the canonical CSR form to caller-owned host arrays:
 * row_ptr [nlat_out+1], in_lat [nnz], lon_off [nnz] (in [0, nlon_in)),
 * vals [nnz, K] float64 (zeros kept).  Entries of each output row are sorted
 * by (in_lat, lon_off).  Any pointer may be NULL to skip that array. */
int disco_psi_export(const disco_psi* psi, int64_t* row_ptr, int32_t* in_lat,
                     int32_t* lon_off, double* vals);

/* Copy the device form of Psi to the current HIP device (allocates device
 * memory owned by the handle).  Must be called before any compute entry point
 * uses the handle.  Calling it again on the same device does nothing;
 * EINVAL if the handle already lives on another device. */
int disco_psi_to_device(disco_psi* psi);

/* Free host and device memory of the handle, including its workspace (it
 * waits for the last call that used the workspace).  NULL is ignored.  The
 * caller must make sure no enqueued work still uses the handle's tables. */
void disco_psi_free(disco_psi* psi);

/* Sparse contraction (the inner sum of the forward equation):
 *   xk[b,c,k,j,q] = sum_{(i,p)} Psi[k,j,(i,p)] * x[b,c,i,(q*s+p) mod nlon_in]
 * x: [B, C, nlat_in, nlon_in] of x_dtype; xk: [B, C, K, nlat_out, nlon_out]
 * of xk_dtype. */
int disco_contract(const disco_psi* psi, const void* x, int x_dtype,
                   void* xk, int xk_dtype, int32_t B, int32_t C, void* stream);

/* Channel/basis contraction (the outer sums of the forward equation):
 *   y[b,co,j,q] = bias[co] + sum_{ci'<Ci/G} sum_k w[co,ci',k] * xk[b, G(co)*Ci/G + ci', k, j, q]
 * with G(co) = co / (Co/G).  EINVAL unless groups divides Ci and Co
 * (DistributedSpectralConvS2 source on the pages raises ValueError for the
 * same condition).  bf16 xk and w with one group of 64 or 128 output
 * channels, Ci*K a multiple of 32 (at least 160 at Co = 128, 192 at Co = 64)
 * and nlat_out*nlon_out a multiple of 8 and at least 256 take a persistent
 * matrix-core kernel that fills one workgroup per compute unit; the
 * environment variable DISCO_EINSUM_PATH=stream selects the double-buffered
 * kernel instead (same sums, float32 accumulation in another order). */
int disco_einsum(const void* xk, int xk_dtype, const void* w, int w_dtype,
                 const float* bias, void* y, int y_dtype,
                 int32_t B, int32_t Ci, int32_t Co, int32_t groups, int32_t K,
                 int32_t nlat_out, int32_t nlon_out, void* stream);

/* Fused forward (DiscreteContinuousConvS2 page, `fused` parameter): the same
 * result as disco_contract followed by disco_einsum, without storing xk in
 * device memory.  x_dtype and w_dtype must be equal.
 *
 * Some layers run in the longitude-spectral form: the forward equation's
 * longitude shift makes each window a circular correlation, so it is
 * evaluated with real DFTs along longitude (a forward transform, the window
 * and channel/basis sums per frequency, an inverse transform), in a
 * workspace of B*Ci*nlat_in*MP*E + B*Co*nlat_out*MP*E bytes with MP =
 * N_in/2 + 1 rounded up to 32 and E = 4 (bf16 spectra) or 8 (float32
 * spectra).
 *
 * Workspace (this call and disco_fused_bwd): the handle keeps one device
 * buffer, allocated with hipMalloc on first need, grown to the largest
 * request and freed by disco_psi_free.  A call that uses it on a stream
 * other than the previous user's first waits for that user's completion
 * event, so calls through one handle are ordered across streams (use one
 * handle per stream for concurrency).  While the stream is being captured
 * into a HIP graph the call takes stream-ordered memory instead
 * (hipMallocAsync / hipFreeAsync nodes that the graph owns).  They are, with N = nlon_in even, N/2 a product of 2, 3
 * and 5 and N <= 1800, groups == 1 and K <= 8:
 *  - bf16 x and w, Ci a multiple of 32, Co 64 or 128, at most 16 input rows
 *    per output row, and stride 1, or stride 2 with N = 720 or 1440 (the
 *    stride-2 output is the stride-1 correlation at every second longitude,
 *    its spectrum folded onto the output grid's frequencies);
 *  - float32 x and w, stride 1, Co <= 128 (both sums on the vector ALUs).
 * The environment variable DISCO_FUSED_PATH=toeplitz selects the direct
 * kernels for them instead.  Rows with 9 to 16 windows (input rows per
 * output row) are summed in two halves of their windows on the 8-window
 * matrix-core kernel when every row has at least two windows;
 * DISCO_SPEC_HALVES=0 selects the 16-window kernel for them instead (same
 * sums, one workgroup per compute unit).  Other layers run the direct kernels: the
 * matrix-core kernel for bf16 layers it accepts, the vector kernels
 * otherwise. */
int disco_fused_fwd(const disco_psi* psi, const void* x, int x_dtype,
                    const void* w, int w_dtype, const float* bias,
                    void* y, int y_dtype, int32_t B, int32_t Ci, int32_t Co,
                    int32_t groups, void* stream);

/* The same result as disco_fused_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): this call allocates nothing.  It always takes the
 * direct algorithms (the matrix-core kernel for the bf16 layers it accepts,
 * the vector kernels otherwise; never the longitude-spectral one, whose
 * workspace grows with the grid), and puts the matrix-core kernel's weight
 * fragments (Ci * Co * 16 bytes) in a fixed 4 MiB device array of the
 * library, held on each device it runs on until the process ends.  EINVAL,
 * before any launch, when a layer needs more than those 4 MiB.  Every call
 * on one device shares that array, so calls that overlap on one device
 * (different streams, or other threads) race and must be ordered by the
 * caller. */
int disco_fused_fwd_noalloc(const disco_psi* psi, const void* x, int x_dtype,
                            const void* w, int w_dtype, const float* bias,
                            void* y, int y_dtype, int32_t B, int32_t Ci, int32_t Co,
                            int32_t groups, void* stream);

/* 1 if disco_fused_fwd with these arguments takes the longitude-spectral
 * path described above, 0 if it takes a direct kernel, negative on error
 * (NULL handle or handle not uploaded).  Reads DISCO_FUSED_PATH like the call
 * itself. */
int disco_fused_is_spectral(const disco_psi* psi, int x_dtype, int32_t Ci, int32_t Co,
                            int32_t groups);

/* ---- Gradients ----------------------------------------------------------
 * The layer trains by backpropagation, and its fused mode recomputes the
 * K-expanded intermediate in the backward pass instead of storing it
 * (DiscreteContinuousConvS2 page, `fused` parameter); with fused=False that
 * intermediate is saved for backward (DistributedDiscreteContinuousConvS2
 * page, `fused` parameter).  The forward equation is linear in x and in w, so
 * the gradients below are the adjoints of its two linear maps.  gy is the
 * gradient of the loss with respect to y, [B, Co, nlat_out, nlon_out].  All
 * sums are accumulated in float32; sums over points run in a fixed order, so
 * results are reproducible.  Work is enqueued on `stream`; disco_fused_bwd
 * takes its scratch from the handle's workspace (described at
 * disco_fused_fwd), disco_einsum_grad_w stream-ordered on that stream. */

/* Adjoint of disco_contract:
 *   gx[b,c,i,n] = sum over (j, q, p) with (q*s + p) mod nlon_in = n of
 *                 sum_k Psi[k,j,(i,p)] * gxk[b,c,k,j,q]
 * gxk: [B, C, K, nlat_out, nlon_out] of gxk_dtype; gx: [B, C, nlat_in,
 * nlon_in] of gx_dtype, overwritten.  Each input row is gathered from the
 * windows that reach it (no atomics).  EUNSUPPORTED when K rows of one
 * output row (K * nlon_out floats) exceed 64 KiB. */
int disco_contract_transpose(const disco_psi* psi, const void* gxk, int gxk_dtype, void* gx,
                             int gx_dtype, int32_t B, int32_t C, void* stream);

/* Adjoint of disco_einsum in xk:
 *   gxk[b, G*Ci/G + ci', k, j, q] = sum_{co in group G} w[co,ci',k] * gy[b,co,j,q]
 * gy [B, Co, nlat_out, nlon_out], w [Co, Ci/groups, K], gxk [B, Ci, K,
 * nlat_out, nlon_out]; any dtype combination. */
int disco_einsum_grad_xk(const void* gy, int gy_dtype, const void* w, int w_dtype, void* gxk,
                         int gxk_dtype, int32_t B, int32_t Ci, int32_t Co, int32_t groups,
                         int32_t K, int32_t nlat_out, int32_t nlon_out, void* stream);

/* Adjoint of disco_einsum in w:
 *   gw[co,ci',k] = sum_{b,j,q} gy[b,co,j,q] * xk[b, G(co)*Ci/G + ci', k, j, q]
 * xk [B, Ci, K, nlat_out, nlon_out] (the saved intermediate), gy [B, Co,
 * nlat_out, nlon_out]; gw [Co, Ci/groups, K] float32, overwritten (zeros for
 * B = 0).  Partial sums over chunks of points, then one reduction.  A bf16
 * gy with groups == 1 and nlon_out a multiple of 8 takes the partial sums
 * on the matrix cores, a float32 xk rounded to bf16 as it is read (the
 * bf16 bar); otherwise they run in float32 on the vector ALUs.  The same
 * holds for disco_fused_bwd's gw. */
int disco_einsum_grad_w(const void* xk, int xk_dtype, const void* gy, int gy_dtype, float* gw,
                        int32_t B, int32_t Ci, int32_t Co, int32_t groups, int32_t K,
                        int32_t nlat_out, int32_t nlon_out, void* stream);

/* Fused-mode backward: from x, w and gy, any of
 *   gx    [B, Ci, nlat_in, nlon_in] of gx_dtype = contract^T(einsum_grad_xk(gy, w)),
 *   gw    [Co, Ci/groups, K] float32            = einsum_grad_w(contract(x), gy),
 *   gbias [Co] float32                          = sum_{b,j,q} gy[b,co,j,q],
 * each overwritten; a NULL pointer skips that gradient (not all three).
 * X_K is recomputed in float32, in slabs of at most ceil(nlat_out / 8)
 * output rows (one slab when the layer's two slab tensors take at most
 * 64 MiB), so neither K-expanded tensor is ever held whole.  The exception
 * is gw of a bf16 layer with a bf16 gy and groups == 1 that the matrix-core
 * contraction takes (Ci a multiple of 32, K <= 8, stride 1 or 2, nlon_in and
 * nlon_out multiples of 8, x and gy 16-byte aligned): its X_K is recomputed
 * whole in bf16 on the matrix cores (at most 4 GiB, in the handle's
 * workspace, which keeps it between calls) and grad_w sums it there (the
 * bf16 bar).  Layers on the longitude-spectral path's tables (stride 1, or stride 2 at
 * 720 or 1440 input longitudes) with bf16 x, w and gy, groups == 1, Ci 64 or
 * 128 and Co a multiple of 32 take gx on the longitude-spectral kernels
 * instead: the adjoint of each window's circular correlation is a circular
 * convolution, so gx = irfft(sum over output rows and k of Psi_hat * sum_co
 * w * rfft(gy)) (at stride 2 gy with a zero inserted after each sample),
 * with bf16 spectra and float32 accumulation (the bf16 bar, not float32
 * exactness); DISCO_FUSED_PATH=toeplitz selects the float32 path for them.
 * Float32 stride-1 layers with a float32 gy (groups == 1, Ci <= 128) take
 * gx on the float32 spectral kernels (float32 spectra, the float32 bar).
 * Layers with one input channel per group take gx with the weights folded
 * into the taps (gy contracted directly, no grad_xk), in float32, and, at
 * stride 1 or 2 with K <= 32, gw with no X_K at all: per window the
 * correlation of gy's output row with x's input row, folded with the
 * window's Psi values, in float32. */
int disco_fused_bwd(const disco_psi* psi, const void* x, int x_dtype, const void* w, int w_dtype,
                    const void* gy, int gy_dtype, void* gx, int gx_dtype, float* gw, float* gbias,
                    int32_t B, int32_t Ci, int32_t Co, int32_t groups, void* stream);

/* Per-kernel timing, for benchmarks and profiling (not part of the pages'
 * method).  With enable != 0, every kernel the library launches from then on
 * is bracketed by a pair of HIP events recorded on its launch stream; with 0,
 * no further events are recorded.  Always returns DISCO_OK. */
int disco_kernel_timing(int enable);

/* Drains the recorded event pairs (waiting for each to complete) into totals
 * per kernel, in order of first launch: kernel i's name is the i-th
 * NUL-terminated string packed into names[0 .. names_len), total_ms[i] its
 * summed event time and launches[i] its launch count.  Returns the number of
 * kernels (0 if nothing was recorded), or DISCO_EINVAL if the buffers are too
 * small (the records are then discarded), or DISCO_EHIP. */
int disco_kernel_timing_read(char* names, int32_t names_len, double* total_ms,
                             int64_t* launches, int32_t max_kernels);

/* Message for the last failed call on this thread ("" if none). */
const char* disco_last_error(void);

/* Library version string. */
const char* disco_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DISCO_H */
