"""GPU parity on the other latitude grids the pages name for grid_in /
grid_out (DistributedSpectralConvS2 page: "legendre-gauss", "lobatto",
"equiangular-trapezoidal"), through the C ABI, against the float64 oracle.

The grid only changes Psi (nodes and quadrature weights, built on the host);
the device kernels are the ones the equiangular grid uses.  Each case runs
the fused forward on the path the library picks (the longitude-spectral one
for the stride-1 cases), the direct kernels where that is spectral or the
layer is bf16, and the unfused contraction + einsum.  Bars as elsewhere: relative L2 <= 1e-5 for
float32, <= 2e-2 for bf16 inputs.
"""
import sys

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def sdc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import spherical_disco_convolution_amd as m
    return m


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# (grid_in, grid_out, B, Ci, Co, nlat_in, nlon_in, nlat_out, nlon_out, kernel_shape, cutoff, dtype,
#  takes the spectral path)
CASES = [
    ("legendre-gauss", "legendre-gauss", 1, 64, 64, 32, 64, 32, 64, (3, 3), 0.3, "bf16", True),
    ("lobatto", "lobatto", 2, 32, 128, 33, 60, 33, 60, (3,), 0.3, "bf16", True),
    ("equiangular-trapezoidal", "equiangular-trapezoidal", 1, 32, 64, 33, 64, 33, 64, (2, 2), 0.25,
     "bf16", True),
    ("legendre-gauss", "equiangular", 1, 4, 6, 48, 96, 25, 48, (3, 3), 0.5, "f32", False),
    ("lobatto", "legendre-gauss", 2, 3, 5, 17, 32, 16, 32, (3,), 0.6, "f32", True),
    # a cap narrower than the input spacing: output rows 0 and 16 (the poles)
    # have no input row in reach, so no windows and an all-zero output row;
    # bf16 takes the direct kernel, float32 the vector spectral one
    ("legendre-gauss", "equiangular", 1, 32, 64, 16, 32, 17, 32, (3, 3), 0.12, "bf16", False),
    ("legendre-gauss", "equiangular", 1, 4, 8, 16, 32, 17, 32, (3, 3), 0.12, "f32", True),
]


def _inputs(case, seed=7):
    gin, gout, B, Ci, Co, nli, nfi, nlo, nfo, ks, cut, dt, _ = case
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, Ci, nli, nfi)).astype(np.float32)
    K = oracle.num_basis(ks)
    w = (rng.standard_normal((Co, Ci, K)) / np.sqrt(Ci * K)).astype(np.float32)
    if dt == "bf16":
        x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
        w = torch.from_numpy(w).to(torch.bfloat16).float().numpy()
    return x, w


def _dev(a, dt):
    t = torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    return t.to(torch.bfloat16) if dt == "bf16" else t


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}-{c[11]}-{c[10]}" for c in CASES])
def test_other_grids_forward(sdc, case, monkeypatch):
    gin, gout, B, Ci, Co, nli, nfi, nlo, nfo, ks, cut, dt, spectral = case
    _say("grid", gin, gout, dt)
    monkeypatch.delenv("DISCO_FUSED_PATH", raising=False)
    x, w = _inputs(case)
    desc = oracle.Desc(nli, nfi, nlo, nfo, tuple(ks), cut, grid_in=gin, grid_out=gout)
    ref = oracle.forward(desc, x, w, 1)
    psi = sdc.psi_build(nli, nfi, nlo, nfo, ks, cut, grid_in=gin, grid_out=gout).to_device()
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    assert sdc.fused_is_spectral(psi, tdt, Ci, Co, 1) == spectral
    xd, wd = _dev(x, dt), _dev(w, dt)
    y = sdc.fused_fwd(psi, xd, wd).float().cpu().numpy()
    err = rel_l2(y, ref)
    _say(f"  fused ({'spectral' if spectral else 'direct'}) rel-L2 {err:.3e}")
    assert err <= TOL[dt]
    # output rows with no support are exactly zero (no bias here)
    empty = ~np.any(ref != 0.0, axis=(0, 1, 3))
    assert np.all(y[:, :, empty, :] == 0.0)
    if spectral or dt == "bf16":
        # the direct kernels on the same layer
        monkeypatch.setenv("DISCO_FUSED_PATH", "toeplitz")
        yt = sdc.fused_fwd(psi, xd, wd).float().cpu().numpy()
        assert rel_l2(yt, ref) <= TOL[dt]
        monkeypatch.delenv("DISCO_FUSED_PATH")
    yu = sdc.einsum(sdc.contract(psi, xd), wd).float().cpu().numpy()
    assert rel_l2(yu, ref) <= TOL[dt]
