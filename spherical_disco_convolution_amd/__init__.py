"""Python binding of libdisco.so, the gfx950 forward DISCO convolution on S^2.

Thin ctypes layer: it marshals torch tensors (device memory and the current
HIP stream) into the C-ABI calls declared in include/disco.h and turns status
codes into exceptions.  All arithmetic runs in the library's HIP kernels;
there is no Python or CPU fallback, and importing fails loudly when the
library is missing.

Entry points (same names as the C ABI, without the ``disco_`` prefix):
    psi_build(...)      -> Psi          host float64 build of the sparse tensor
    contract(psi, x)    -> xk           [B, C, K, nlat_out, nlon_out]
    einsum(xk, w, ...)  -> y            [B, Co, nlat_out, nlon_out]
    fused_fwd(psi, x, w, ...) -> y      same result without storing xk
  gradients (gy: gradient of the loss with respect to y):
    contract_transpose(psi, gxk) -> gx          adjoint of contract
    einsum_grad_xk(gy, w, ...)   -> gxk         adjoint of einsum in xk
    einsum_grad_w(xk, gy, ...)   -> gw          adjoint of einsum in w
    fused_bwd(psi, x, w, gy, ...) -> (gx, gw, gbias)   X_K recomputed, never whole
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdisco.so")

DISCO_OK = 0
DISCO_EINVAL = -1
DISCO_EUNSUPPORTED = -2
DISCO_ENOMEM = -3
DISCO_EHIP = -4

F32 = 0
BF16 = 1

GRIDS = {"equiangular": 0, "legendre-gauss": 1, "lobatto": 2, "equiangular-trapezoidal": 3}
BASES = {"piecewise linear": 0}
NORMS = {"none": 0}


class _Desc(ctypes.Structure):
    _fields_ = [
        ("nlat_in", ctypes.c_int32), ("nlon_in", ctypes.c_int32),
        ("nlat_out", ctypes.c_int32), ("nlon_out", ctypes.c_int32),
        ("grid_in", ctypes.c_int32), ("grid_out", ctypes.c_int32),
        ("basis_type", ctypes.c_int32), ("basis_norm", ctypes.c_int32),
        ("kernel_shape", ctypes.c_int32 * 2),
        ("theta_cutoff", ctypes.c_double),
    ]


def _load():
    # PyTorch ships its own HIP runtime (SONAME libamdhip64.so.7).  Loading
    # torch first makes libdisco.so bind to that same runtime, so the device
    # pointers and stream handles torch hands over are valid in the library.
    # Loading libdisco.so first would pull in a second HIP runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python spherical_disco_convolution_amd/build_lib.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    sig = {
        "disco_psi_build": (ctypes.c_int, [ctypes.POINTER(_Desc), ctypes.POINTER(P)]),
        "disco_psi_query": (ctypes.c_int, [P, ctypes.POINTER(I32), ctypes.POINTER(I64),
                                           ctypes.POINTER(I64), ctypes.POINTER(D)]),
        "disco_psi_export": (ctypes.c_int, [P, P, P, P, P]),
        "disco_psi_to_device": (ctypes.c_int, [P]),
        "disco_psi_free": (None, [P]),
        "disco_contract": (ctypes.c_int, [P, P, ctypes.c_int, P, ctypes.c_int, I32, I32, P]),
        "disco_einsum": (ctypes.c_int, [P, ctypes.c_int, P, ctypes.c_int, P, P, ctypes.c_int,
                                        I32, I32, I32, I32, I32, I32, I32, P]),
        "disco_fused_fwd": (ctypes.c_int, [P, P, ctypes.c_int, P, ctypes.c_int, P, P,
                                           ctypes.c_int, I32, I32, I32, I32, P]),
        "disco_fused_fwd_noalloc": (ctypes.c_int, [P, P, ctypes.c_int, P, ctypes.c_int, P, P,
                                                   ctypes.c_int, I32, I32, I32, I32, P]),
        "disco_fused_is_spectral": (ctypes.c_int, [P, ctypes.c_int, I32, I32, I32]),
        "disco_contract_transpose": (ctypes.c_int, [P, P, ctypes.c_int, P, ctypes.c_int, I32, I32,
                                                    P]),
        "disco_einsum_grad_xk": (ctypes.c_int, [P, ctypes.c_int, P, ctypes.c_int, P, ctypes.c_int,
                                                I32, I32, I32, I32, I32, I32, I32, P]),
        "disco_einsum_grad_w": (ctypes.c_int, [P, ctypes.c_int, P, ctypes.c_int, P, I32, I32, I32,
                                               I32, I32, I32, I32, P]),
        "disco_fused_bwd": (ctypes.c_int, [P, P, ctypes.c_int, P, ctypes.c_int, P, ctypes.c_int, P,
                                           ctypes.c_int, P, P, I32, I32, I32, I32, P]),
        "disco_kernel_timing": (ctypes.c_int, [ctypes.c_int]),
        "disco_kernel_timing_read": (ctypes.c_int, [ctypes.c_char_p, I32, ctypes.POINTER(D),
                                                    ctypes.POINTER(I64), I32]),
        "disco_last_error": (ctypes.c_char_p, []),
        "disco_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("disco_psi_build", "disco_psi_query", "disco_psi_export", "disco_psi_to_device",
            "disco_psi_free", "disco_contract", "disco_einsum", "disco_fused_fwd",
            "disco_fused_fwd_noalloc",
            "disco_fused_is_spectral", "disco_contract_transpose", "disco_einsum_grad_xk",
            "disco_einsum_grad_w", "disco_fused_bwd", "disco_kernel_timing", "disco_kernel_timing_read",
            "disco_last_error", "disco_version")


def version() -> str:
    return _lib.disco_version().decode()


def _check(rc: int, what: str):
    if rc == DISCO_OK:
        return
    msg = f"{what}: {_lib.disco_last_error().decode()}"
    if rc == DISCO_EINVAL:
        raise ValueError(msg)
    if rc == DISCO_EUNSUPPORTED:
        raise NotImplementedError(msg)
    if rc == DISCO_ENOMEM:
        raise MemoryError(msg)
    raise RuntimeError(msg)


def _kernel_shape(ks):
    if isinstance(ks, int):
        return (ks, 0)
    ks = tuple(int(v) for v in ks)
    if len(ks) == 1:
        return (ks[0], 0)
    if len(ks) == 2:
        return ks
    raise ValueError(f"kernel_shape must be an int or a tuple of one or two ints, got {ks}")


class Psi:
    """Handle of a built Psi tensor (library-owned)."""

    def __init__(self, handle, desc: _Desc):
        self._h = ctypes.c_void_p(handle)
        self.desc = desc
        K = ctypes.c_int32()
        nnz = ctypes.c_int64()
        nzz = ctypes.c_int64()
        cut = ctypes.c_double()
        _check(_lib.disco_psi_query(self._h, ctypes.byref(K), ctypes.byref(nnz),
                                    ctypes.byref(nzz), ctypes.byref(cut)), "psi_query")
        self.K = K.value
        self.nnz = nnz.value
        self.nnz_nonzero = nzz.value
        self.theta_cutoff = cut.value
        self.nlat_in, self.nlon_in = desc.nlat_in, desc.nlon_in
        self.nlat_out, self.nlon_out = desc.nlat_out, desc.nlon_out
        self.on_device = False

    @property
    def handle(self):
        return self._h

    def export(self):
        """Canonical CSR as numpy arrays (row_ptr, in_lat, lon_off, vals[nnz, K])."""
        row_ptr = np.zeros(self.nlat_out + 1, dtype=np.int64)
        in_lat = np.zeros(self.nnz, dtype=np.int32)
        lon_off = np.zeros(self.nnz, dtype=np.int32)
        vals = np.zeros((self.nnz, self.K), dtype=np.float64)
        _check(_lib.disco_psi_export(self._h, row_ptr.ctypes.data, in_lat.ctypes.data,
                                     lon_off.ctypes.data, vals.ctypes.data), "psi_export")
        return row_ptr, in_lat, lon_off, vals

    def to_device(self):
        """Copy the device form to the current HIP device (once)."""
        _check(_lib.disco_psi_to_device(self._h), "psi_to_device")
        self.on_device = True
        return self

    def __del__(self):
        h = getattr(self, "_h", None)
        # at interpreter exit the module's globals may already be cleared:
        # the process is ending and the handle goes with it
        if h is not None and h.value and _lib is not None:
            _lib.disco_psi_free(h)
            self._h = ctypes.c_void_p(0)


def psi_build(nlat_in: int, nlon_in: int, nlat_out: int, nlon_out: int, kernel_shape,
              theta_cutoff: float | None = None, grid_in: str = "equiangular",
              grid_out: str = "equiangular", basis_type: str = "piecewise linear",
              basis_norm_mode: str = "none") -> Psi:
    """Build Psi on the host (float64).  Arguments follow the layer's
    constructor: in_shape/out_shape as (nlat, nlon), kernel_shape, theta_cutoff
    (None selects (nr+1)*pi/(nlat_out-1)), grids, basis type and norm."""
    d = _Desc()
    d.nlat_in, d.nlon_in, d.nlat_out, d.nlon_out = nlat_in, nlon_in, nlat_out, nlon_out
    for key, table, val in (("grid_in", GRIDS, grid_in), ("grid_out", GRIDS, grid_out),
                            ("basis_type", BASES, basis_type), ("basis_norm", NORMS, basis_norm_mode)):
        if val not in table:
            raise NotImplementedError(f"{key}={val!r} is not implemented (supported: {list(table)})")
        setattr(d, key, table[val])
    nr, nphi = _kernel_shape(kernel_shape)
    d.kernel_shape[0], d.kernel_shape[1] = nr, nphi
    if theta_cutoff is None:
        d.theta_cutoff = 0.0
    else:
        if not (theta_cutoff > 0.0):
            raise ValueError(f"theta_cutoff must be positive, got {theta_cutoff}")
        d.theta_cutoff = float(theta_cutoff)
    h = ctypes.c_void_p()
    _check(_lib.disco_psi_build(ctypes.byref(d), ctypes.byref(h)), "psi_build")
    return Psi(h.value, d)


# ----------------------------------------------------------------------------
# compute entry points (torch tensors on the current HIP device)
# ----------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _torch_dtype(code: int):
    torch = _torch()
    return torch.float32 if code == F32 else torch.bfloat16


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def contract(psi: Psi, x, xk=None, xk_dtype=None, stream=None):
    """xk[b,c,k,j,q] = sum_(i,p) Psi[k,j,(i,p)] x[b,c,i,(q*s+p) mod nlon_in]."""
    torch = _torch()
    if x.dim() != 4:
        raise ValueError("x must be [B, C, nlat_in, nlon_in]")
    B, C = x.shape[:2]
    _need(x, "x", (B, C, psi.nlat_in, psi.nlon_in))
    if xk is None:
        dt = x.dtype if xk_dtype is None else xk_dtype
        xk = torch.empty((B, C, psi.K, psi.nlat_out, psi.nlon_out), dtype=dt, device=x.device)
    _need(xk, "xk", (B, C, psi.K, psi.nlat_out, psi.nlon_out))
    _check(_lib.disco_contract(psi.handle, x.data_ptr(), _dtype_code(x), xk.data_ptr(),
                               _dtype_code(xk), B, C, _stream(stream)), "contract")
    return xk


def einsum(xk, w, groups: int = 1, bias=None, y=None, out_dtype=None, stream=None):
    """y[b,co,j,q] = bias[co] + sum_(ci',k) w[co,ci',k] xk[b, G(co)*Ci/G+ci', k, j, q]."""
    torch = _torch()
    if xk.dim() != 5 or w.dim() != 3:
        raise ValueError("xk must be [B, Ci, K, nlat_out, nlon_out] and w [Co, Ci/groups, K]")
    B, Ci, K, H, W = xk.shape
    Co = w.shape[0]
    _need(xk, "xk", (B, Ci, K, H, W))
    if groups < 1 or Ci % groups or Co % groups:
        raise ValueError(f"groups ({groups}) must divide in_channels ({Ci}) and out_channels ({Co})")
    _need(w, "w", (Co, Ci // groups, K))
    if y is None:
        dt = torch.float32 if out_dtype is None else out_dtype
        y = torch.empty((B, Co, H, W), dtype=dt, device=xk.device)
    _need(y, "y", (B, Co, H, W))
    bptr = None
    if bias is not None:
        _need(bias, "bias", (Co,))
        if bias.dtype != torch.float32:
            raise ValueError("bias must be float32")
        bptr = bias.data_ptr()
    _check(_lib.disco_einsum(xk.data_ptr(), _dtype_code(xk), w.data_ptr(), _dtype_code(w), bptr,
                             y.data_ptr(), _dtype_code(y), B, Ci, Co, groups, K, H, W,
                             _stream(stream)), "einsum")
    return y


def fused_is_spectral(psi: Psi, x_dtype, Ci: int, Co: int, groups: int = 1) -> bool:
    """Whether fused_fwd takes the longitude-spectral path for these arguments
    (x_dtype: a torch dtype)."""
    torch = _torch()
    code = BF16 if x_dtype == torch.bfloat16 else F32
    rc = _lib.disco_fused_is_spectral(psi.handle, code, Ci, Co, groups)
    if rc < 0:
        _check(rc, "fused_is_spectral")
    return rc == 1


def kernel_timing(enable: bool) -> None:
    """Start (True) or stop (False) recording a HIP event pair around every
    kernel the library launches, on its launch stream."""
    _check(_lib.disco_kernel_timing(1 if enable else 0), "kernel_timing")


def kernel_timing_read(max_kernels: int = 64) -> dict:
    """Drain the recorded events: {kernel name: (total milliseconds, launches)},
    in order of first launch.  Waits for the recorded launches to finish."""
    names = ctypes.create_string_buffer(64 * max_kernels)
    tot = (ctypes.c_double * max_kernels)()
    cnt = (ctypes.c_int64 * max_kernels)()
    n = _lib.disco_kernel_timing_read(names, len(names), tot, cnt, max_kernels)
    if n < 0:
        _check(n, "kernel_timing_read")
    out, off = {}, 0
    raw = names.raw
    for i in range(n):
        end = raw.index(b"\0", off)
        out[raw[off:end].decode()] = (tot[i], cnt[i])
        off = end + 1
    return out


def fused_fwd(psi: Psi, x, w, groups: int = 1, bias=None, y=None, out_dtype=None, stream=None):
    """The forward DISCO convolution without storing the K-expanded tensor."""
    torch = _torch()
    if x.dim() != 4 or w.dim() != 3:
        raise ValueError("x must be [B, Ci, nlat_in, nlon_in] and w [Co, Ci/groups, K]")
    B, Ci = x.shape[:2]
    Co = w.shape[0]
    _need(x, "x", (B, Ci, psi.nlat_in, psi.nlon_in))
    if groups < 1 or Ci % groups or Co % groups:
        raise ValueError(f"groups ({groups}) must divide in_channels ({Ci}) and out_channels ({Co})")
    _need(w, "w", (Co, Ci // groups, psi.K))
    if y is None:
        dt = torch.float32 if out_dtype is None else out_dtype
        y = torch.empty((B, Co, psi.nlat_out, psi.nlon_out), dtype=dt, device=x.device)
    _need(y, "y", (B, Co, psi.nlat_out, psi.nlon_out))
    bptr = None
    if bias is not None:
        _need(bias, "bias", (Co,))
        if bias.dtype != torch.float32:
            raise ValueError("bias must be float32")
        bptr = bias.data_ptr()
    _check(_lib.disco_fused_fwd(psi.handle, x.data_ptr(), _dtype_code(x), w.data_ptr(),
                                _dtype_code(w), bptr, y.data_ptr(), _dtype_code(y), B, Ci, Co,
                                groups, _stream(stream)), "fused_fwd")
    return y



def fused_fwd_noalloc(psi: Psi, x, w, y, groups: int = 1, bias=None, stream=None):
    """fused_fwd for callers that cannot allocate device memory: the direct
    algorithms with the library's fixed scratch; y must be given."""
    if x.dim() != 4 or w.dim() != 3:
        raise ValueError("x must be [B, Ci, nlat_in, nlon_in] and w [Co, Ci/groups, K]")
    B, Ci = x.shape[:2]
    Co = w.shape[0]
    _need(x, "x", (B, Ci, psi.nlat_in, psi.nlon_in))
    if groups < 1 or Ci % groups or Co % groups:
        raise ValueError(f"groups ({groups}) must divide in_channels ({Ci}) and out_channels ({Co})")
    _need(w, "w", (Co, Ci // groups, psi.K))
    _need(y, "y", (B, Co, psi.nlat_out, psi.nlon_out))
    bptr = None
    if bias is not None:
        _need(bias, "bias", (Co,))
        bptr = bias.data_ptr()
    _check(_lib.disco_fused_fwd_noalloc(psi.handle, x.data_ptr(), _dtype_code(x), w.data_ptr(),
                                        _dtype_code(w), bptr, y.data_ptr(), _dtype_code(y), B, Ci,
                                        Co, groups, _stream(stream)), "fused_fwd_noalloc")
    return y


# ----------------------------------------------------------------------------
# gradients
# ----------------------------------------------------------------------------
def contract_transpose(psi: Psi, gxk, gx=None, gx_dtype=None, stream=None):
    """gx[b,c,i,(q*s+p) mod nlon_in] = sum over windows of Psi[k,j,(i,p)] gxk[b,c,k,j,q]
    (the adjoint of contract)."""
    torch = _torch()
    if gxk.dim() != 5:
        raise ValueError("gxk must be [B, C, K, nlat_out, nlon_out]")
    B, C = gxk.shape[:2]
    _need(gxk, "gxk", (B, C, psi.K, psi.nlat_out, psi.nlon_out))
    if gx is None:
        dt = torch.float32 if gx_dtype is None else gx_dtype
        gx = torch.empty((B, C, psi.nlat_in, psi.nlon_in), dtype=dt, device=gxk.device)
    _need(gx, "gx", (B, C, psi.nlat_in, psi.nlon_in))
    _check(_lib.disco_contract_transpose(psi.handle, gxk.data_ptr(), _dtype_code(gxk),
                                         gx.data_ptr(), _dtype_code(gx), B, C, _stream(stream)),
           "contract_transpose")
    return gx


def einsum_grad_xk(gy, w, groups: int = 1, gxk=None, out_dtype=None, stream=None):
    """gxk[b, G*Ci/G+ci', k, j, q] = sum_{co in G} w[co,ci',k] gy[b,co,j,q]."""
    torch = _torch()
    if gy.dim() != 4 or w.dim() != 3:
        raise ValueError("gy must be [B, Co, nlat_out, nlon_out] and w [Co, Ci/groups, K]")
    B, Co, H, W = gy.shape
    _need(gy, "gy", (B, Co, H, W))
    if groups < 1 or Co % groups or w.shape[0] != Co:
        raise ValueError(f"w must have {Co} rows and groups ({groups}) must divide them")
    Ci, K = w.shape[1] * groups, w.shape[2]
    _need(w, "w", (Co, Ci // groups, K))
    if gxk is None:
        dt = torch.float32 if out_dtype is None else out_dtype
        gxk = torch.empty((B, Ci, K, H, W), dtype=dt, device=gy.device)
    _need(gxk, "gxk", (B, Ci, K, H, W))
    _check(_lib.disco_einsum_grad_xk(gy.data_ptr(), _dtype_code(gy), w.data_ptr(), _dtype_code(w),
                                     gxk.data_ptr(), _dtype_code(gxk), B, Ci, Co, groups, K, H, W,
                                     _stream(stream)), "einsum_grad_xk")
    return gxk


def einsum_grad_w(xk, gy, groups: int = 1, gw=None, stream=None):
    """gw[co,ci',k] = sum_{b,j,q} gy[b,co,j,q] xk[b, G(co)*Ci/G+ci', k, j, q] (float32)."""
    torch = _torch()
    if xk.dim() != 5 or gy.dim() != 4:
        raise ValueError("xk must be [B, Ci, K, nlat_out, nlon_out] and gy [B, Co, nlat_out, nlon_out]")
    B, Ci, K, H, W = xk.shape
    Co = gy.shape[1]
    _need(xk, "xk", (B, Ci, K, H, W))
    _need(gy, "gy", (B, Co, H, W))
    if groups < 1 or Ci % groups or Co % groups:
        raise ValueError(f"groups ({groups}) must divide in_channels ({Ci}) and out_channels ({Co})")
    if gw is None:
        gw = torch.empty((Co, Ci // groups, K), dtype=torch.float32, device=xk.device)
    _need(gw, "gw", (Co, Ci // groups, K))
    if gw.dtype != torch.float32:
        raise ValueError("gw must be float32")
    _check(_lib.disco_einsum_grad_w(xk.data_ptr(), _dtype_code(xk), gy.data_ptr(), _dtype_code(gy),
                                    gw.data_ptr(), B, Ci, Co, groups, K, H, W, _stream(stream)),
           "einsum_grad_w")
    return gw


def fused_bwd(psi: Psi, x, w, gy, groups: int = 1, need_gx: bool = True, need_gw: bool = True,
              need_gbias: bool = False, gx_dtype=None, stream=None):
    """Gradients (gx, gw, gbias) of sum(gy * fused_fwd(psi, x, w)) with X_K
    recomputed slab by slab; entries not asked for are None."""
    torch = _torch()
    if x.dim() != 4 or w.dim() != 3 or gy.dim() != 4:
        raise ValueError("x must be [B, Ci, nlat_in, nlon_in], w [Co, Ci/groups, K] and gy "
                         "[B, Co, nlat_out, nlon_out]")
    B, Ci = x.shape[:2]
    Co = w.shape[0]
    _need(x, "x", (B, Ci, psi.nlat_in, psi.nlon_in))
    if groups < 1 or Ci % groups or Co % groups:
        raise ValueError(f"groups ({groups}) must divide in_channels ({Ci}) and out_channels ({Co})")
    _need(w, "w", (Co, Ci // groups, psi.K))
    _need(gy, "gy", (B, Co, psi.nlat_out, psi.nlon_out))
    gx = gw = gb = None
    if need_gx:
        gx = torch.empty((B, Ci, psi.nlat_in, psi.nlon_in),
                         dtype=torch.float32 if gx_dtype is None else gx_dtype, device=x.device)
    if need_gw:
        gw = torch.empty((Co, Ci // groups, psi.K), dtype=torch.float32, device=x.device)
    if need_gbias:
        gb = torch.empty((Co,), dtype=torch.float32, device=x.device)
    _check(_lib.disco_fused_bwd(psi.handle, x.data_ptr(), _dtype_code(x), w.data_ptr(),
                                _dtype_code(w), gy.data_ptr(), _dtype_code(gy),
                                gx.data_ptr() if gx is not None else None,
                                _dtype_code(gx) if gx is not None else F32,
                                gw.data_ptr() if gw is not None else None,
                                gb.data_ptr() if gb is not None else None,
                                B, Ci, Co, groups, _stream(stream)), "fused_bwd")
    return gx, gw, gb
