"""C-ABI checks that need no GPU: every symbol declared in include/*.h is
exported by libdisco.so, and invalid requests are rejected with the right
status and a message before any device work.
"""
import ctypes
import glob
import math
import os
import re
import subprocess
import sys

import pytest

import spherical_disco_convolution_amd as sdc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(disco_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for required in ("disco_psi_build", "disco_contract", "disco_einsum", "disco_fused_fwd"):
        assert required in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(sdc.LIB_PATH)
    out = subprocess.run(["nm", "-D", "--defined-only", sdc.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared_functions():
        assert name in exported, name
        getattr(lib, name)


def _rc_build(**kw):
    d = sdc._Desc()
    vals = dict(nlat_in=33, nlon_in=64, nlat_out=33, nlon_out=64, grid_in=0, grid_out=0,
                basis_type=0, basis_norm=0, theta_cutoff=0.3)
    ks = kw.pop("kernel_shape", (3, 0))
    vals.update(kw)
    for k, v in vals.items():
        setattr(d, k, v)
    d.kernel_shape[0], d.kernel_shape[1] = ks
    h = ctypes.c_void_p()
    rc = sdc._lib.disco_psi_build(ctypes.byref(d), ctypes.byref(h))
    msg = sdc._lib.disco_last_error().decode()
    if rc == 0:
        sdc._lib.disco_psi_free(h)
    return rc, msg


@pytest.mark.parametrize("kw,code", [
    (dict(nlat_in=1), sdc.DISCO_EINVAL),
    (dict(nlat_out=1), sdc.DISCO_EINVAL),
    (dict(nlon_in=0), sdc.DISCO_EINVAL),
    (dict(nlon_out=48), sdc.DISCO_EINVAL),            # 64 % 48 != 0
    (dict(nlon_out=128), sdc.DISCO_EINVAL),           # upsampling in longitude
    (dict(theta_cutoff=math.pi), sdc.DISCO_EINVAL),
    (dict(theta_cutoff=4.0), sdc.DISCO_EINVAL),
    (dict(theta_cutoff=float("nan")), sdc.DISCO_EINVAL),
    (dict(kernel_shape=(0, 0)), sdc.DISCO_EINVAL),
    (dict(kernel_shape=(3, -1)), sdc.DISCO_EINVAL),
    (dict(kernel_shape=(10, 8)), sdc.DISCO_EUNSUPPORTED),   # K = 73 > 64
    (dict(grid_in=4), sdc.DISCO_EUNSUPPORTED),       # unknown grid codes
    (dict(grid_out=-1), sdc.DISCO_EUNSUPPORTED),
    (dict(basis_type=1), sdc.DISCO_EUNSUPPORTED),
    (dict(basis_norm=1), sdc.DISCO_EUNSUPPORTED),
])
def test_build_rejects(kw, code):
    rc, msg = _rc_build(**kw)
    assert rc == code
    assert msg


@pytest.mark.parametrize("gin,gout", [(1, 1), (2, 2), (3, 3), (1, 0), (0, 2), (2, 3)])
def test_build_accepts_every_grid_code(gin, gout):
    # equiangular 0, legendre-gauss 1, lobatto 2, equiangular-trapezoidal 3
    rc, msg = _rc_build(grid_in=gin, grid_out=gout)
    assert rc == 0, msg


def test_build_null_arguments():
    assert sdc._lib.disco_psi_build(None, None) == sdc.DISCO_EINVAL
    assert sdc._lib.disco_psi_query(None, None, None, None, None) == sdc.DISCO_EINVAL
    assert sdc._lib.disco_psi_export(None, None, None, None, None) == sdc.DISCO_EINVAL
    assert sdc._lib.disco_psi_to_device(None) == sdc.DISCO_EINVAL
    sdc._lib.disco_psi_free(None)   # no-op


def test_python_errors():
    with pytest.raises(ValueError):
        sdc.psi_build(33, 64, 33, 48, (3,), 0.3)
    with pytest.raises(NotImplementedError):
        sdc.psi_build(33, 64, 33, 64, (3,), 0.3, grid_in="healpix")
    with pytest.raises(NotImplementedError):
        sdc.psi_build(33, 64, 33, 64, (3,), 0.3, basis_norm_mode="nodal")
    with pytest.raises(ValueError):
        sdc.psi_build(33, 64, 33, 64, (3, 3, 3), 0.3)
    with pytest.raises(ValueError):
        sdc.psi_build(33, 64, 33, 64, (3,), -1.0)


def test_forced_host_allocation_failure():
    code = (
        "import ctypes, spherical_disco_convolution_amd as s\n"
        "d = s._Desc(); d.nlat_in=d.nlat_out=33; d.nlon_in=d.nlon_out=64\n"
        "d.kernel_shape[0]=3; d.theta_cutoff=0.3\n"
        "h = ctypes.c_void_p()\n"
        "print(s._lib.disco_psi_build(ctypes.byref(d), ctypes.byref(h)))\n")
    env = dict(os.environ, DISCO_TEST_FAIL_HOST_ALLOC="1")
    out = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True,
                         text=True, check=True).stdout.strip()
    assert int(out) == sdc.DISCO_ENOMEM


def test_compute_calls_reject_bad_arguments_before_device_work():
    L = sdc._lib
    p = sdc.psi_build(33, 64, 33, 64, (3,), 0.3)
    fake = ctypes.c_void_p(0x1000)
    # unknown dtype codes
    assert L.disco_contract(p.handle, fake, 7, fake, 0, 1, 1, None) == sdc.DISCO_EINVAL
    assert L.disco_einsum(fake, 0, fake, 0, None, fake, 9, 1, 4, 4, 1, 3, 33, 64, None) == sdc.DISCO_EINVAL
    # groups must divide channels (the spectral layer's source raises ValueError for this)
    assert L.disco_einsum(fake, 0, fake, 0, None, fake, 0, 1, 6, 4, 4, 3, 33, 64, None) == sdc.DISCO_EINVAL
    assert "groups" in L.disco_last_error().decode()
    assert L.disco_fused_fwd(p.handle, fake, 0, fake, 0, None, fake, 0, 1, 4, 6, 4, None) == sdc.DISCO_EINVAL
    # negative sizes
    assert L.disco_contract(p.handle, fake, 0, fake, 0, -1, 1, None) == sdc.DISCO_EINVAL
    assert L.disco_einsum(fake, 0, fake, 0, None, fake, 0, 1, 0, 4, 1, 3, 33, 64, None) == sdc.DISCO_EINVAL
    # mixed input dtypes
    assert L.disco_fused_fwd(p.handle, fake, 0, fake, 1, None, fake, 0, 1, 4, 4, 1, None) == sdc.DISCO_EUNSUPPORTED
    # null handle
    assert L.disco_contract(None, fake, 0, fake, 0, 1, 1, None) == sdc.DISCO_EINVAL
    assert L.disco_fused_fwd(None, fake, 0, fake, 0, None, fake, 0, 1, 4, 4, 1, None) == sdc.DISCO_EINVAL
    # empty batch is a no-op
    assert L.disco_contract(p.handle, fake, 0, fake, 0, 0, 4, None) == sdc.DISCO_OK


def test_handle_without_device_copy_is_rejected_or_no_gpu():
    # Without disco_psi_to_device the compute calls must refuse the handle
    # (or, on a machine without a GPU, report the HIP failure); never crash.
    L = sdc._lib
    p = sdc.psi_build(33, 64, 33, 64, (3,), 0.3)
    fake = ctypes.c_void_p(0x1000)
    rc = L.disco_contract(p.handle, fake, 0, fake, 0, 1, 1, None)
    assert rc in (sdc.DISCO_EINVAL, sdc.DISCO_EHIP)
    assert L.disco_last_error().decode()


def test_kernel_timing_host_logic():
    # with nothing launched, a read drains nothing; bad buffers are argument errors
    assert sdc._lib.disco_kernel_timing(1) == 0
    assert sdc.kernel_timing_read() == {}
    assert sdc._lib.disco_kernel_timing(0) == 0
    tot = (ctypes.c_double * 1)()
    cnt = (ctypes.c_int64 * 1)()
    assert sdc._lib.disco_kernel_timing_read(None, 0, tot, cnt, -1) == sdc.DISCO_EINVAL
    assert sdc._lib.disco_kernel_timing_read(None, 16, tot, cnt, 1) == sdc.DISCO_EINVAL
    assert sdc._lib.disco_kernel_timing_read(None, 0, None, None, 0) == 0


def test_backward_argument_errors_before_any_device_work():
    lib = sdc._lib
    P = ctypes.c_void_p
    # NULL handle
    assert lib.disco_contract_transpose(None, None, 0, None, 0, 1, 1, None) == sdc.DISCO_EINVAL
    assert "NULL" in lib.disco_last_error().decode()
    assert lib.disco_fused_bwd(None, None, 0, None, 0, None, 0, None, 0, None, None, 1, 1, 1, 1,
                               None) == sdc.DISCO_EINVAL
    # unknown dtype codes
    assert lib.disco_einsum_grad_w(None, 7, None, 0, None, 1, 4, 4, 1, 3, 2, 2,
                                   None) == sdc.DISCO_EINVAL
    assert lib.disco_einsum_grad_xk(None, 0, None, 9, None, 0, 1, 4, 4, 1, 3, 2, 2,
                                    None) == sdc.DISCO_EINVAL
    # groups must divide both channel counts (the DistributedSpectralConvS2
    # source on the pages raises ValueError for this)
    assert lib.disco_einsum_grad_w(None, 0, None, 0, None, 1, 6, 4, 4, 3, 2, 2,
                                   None) == sdc.DISCO_EINVAL
    assert "groups" in lib.disco_last_error().decode()
    assert lib.disco_einsum_grad_xk(None, 0, None, 0, None, 0, 1, 5, 4, 2, 3, 2, 2,
                                    None) == sdc.DISCO_EINVAL
    # non-positive sizes
    assert lib.disco_einsum_grad_w(None, 0, None, 0, None, -1, 4, 4, 1, 3, 2, 2,
                                   None) == sdc.DISCO_EINVAL
    # a fused backward that asks for nothing
    d = sdc._Desc()
    d.nlat_in, d.nlon_in, d.nlat_out, d.nlon_out = 9, 16, 9, 16
    d.kernel_shape[0], d.kernel_shape[1] = 3, 0
    d.theta_cutoff = 0.7
    h = P()
    assert lib.disco_psi_build(ctypes.byref(d), ctypes.byref(h)) == 0
    try:
        assert lib.disco_fused_bwd(h, None, 0, None, 0, None, 0, None, 0, None, None, 1, 2, 2, 1,
                                   None) == sdc.DISCO_EINVAL
        assert "NULL" in lib.disco_last_error().decode()
        # a handle with no device copy
        assert lib.disco_contract_transpose(h, None, 0, None, 0, 1, 2, None) in (
            sdc.DISCO_EINVAL, sdc.DISCO_EHIP)
    finally:
        lib.disco_psi_free(h)
