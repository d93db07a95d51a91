"""The no-allocation fused forward (disco_fused_fwd_noalloc) through the C ABI,
against disco_fused_fwd on the same inputs, on two calls in a row, the second
with a smaller input; and its rejection of a layer whose weight fragments do
not fit its fixed scratch.

Where disco_fused_fwd takes a direct algorithm too, both run the same
kernels and must agree bit for bit.  Where it takes the longitude-spectral
algorithm, the two are different roundings of the same sums and are held to
the bf16 bar (relative L2 <= 2e-2) against each other and against the
oracle.
"""
import math

import numpy as np
import pytest

import oracle
from disco_workloads import Workload, draw_inputs, round_bf16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


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


def W(name, B, Ci, Co, G, nli, nfi, nlo, nfo, ks, cut, dt, seed=41):
    return Workload(name, seed, B, Ci, Co, G, nli, nfi, nlo, nfo, ks, oracle.num_basis(ks), cut,
                    dt)


def _run(sdc, wl):
    x, w = draw_inputs(wl)
    if wl.dtype == "bf16":
        x, w = round_bf16(x), round_bf16(w)
    tdt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    psi = sdc.psi_build(wl.nlat_in, wl.nlon_in, wl.nlat_out, wl.nlon_out, wl.kernel_shape,
                        wl.theta_cutoff).to_device()
    xd = torch.from_numpy(x).cuda().to(tdt)
    wd = torch.from_numpy(w).cuda().to(tdt)
    y_ref = sdc.fused_fwd(psi, xd, wd, groups=wl.groups)
    y = torch.full_like(y_ref, float("nan"))
    sdc.kernel_timing(True)
    try:
        sdc.fused_fwd_noalloc(psi, xd, wd, y, groups=wl.groups)
        names = set(sdc.kernel_timing_read())
    finally:
        sdc.kernel_timing(False)
    torch.cuda.synchronize()
    d = oracle.Desc(wl.nlat_in, wl.nlon_in, wl.nlat_out, wl.nlon_out, wl.kernel_shape,
                    wl.theta_cutoff)
    ora = oracle.forward(d, x, w, wl.groups)
    spectral = sdc.fused_is_spectral(psi, tdt, wl.Ci, wl.Co, wl.groups)
    return y, y_ref, ora, names, spectral


# pairs of calls in a row, the second with a smaller input
PAIRS = [
    # bf16, stride 2: the direct matrix-core kernel on both entry points
    (W("direct_big", 2, 128, 128, 1, 73, 144, 37, 72, (3, 3), 4 * math.pi / 36, "bf16"),
     W("direct_small", 1, 64, 64, 1, 33, 64, 17, 32, (3, 3), 4 * math.pi / 16, "bf16")),
    # float32 and grouped layers: the vector kernels on both entry points
    (W("f32_big", 2, 16, 8, 2, 33, 64, 33, 64, (3, 3), 4 * math.pi / 32, "f32"),
     W("f32_small", 1, 4, 4, 1, 17, 32, 17, 32, (3,), 0.5, "f32")),
    # bf16, stride 1: disco_fused_fwd takes the spectral algorithm, the
    # no-allocation call the direct one
    (W("stride1_big", 1, 128, 128, 1, 49, 96, 49, 96, (3, 3), 4 * math.pi / 48, "bf16"),
     W("stride1_small", 1, 64, 64, 1, 25, 48, 25, 48, (3, 3), 4 * math.pi / 24, "bf16")),
]


@pytest.mark.parametrize("pair", PAIRS, ids=[p[0].name for p in PAIRS])
def test_noalloc_matches_fused_fwd_twice(sdc, pair):
    for wl in pair:
        y, y_ref, ora, names, spectral = _run(sdc, wl)
        assert not torch.isnan(y).any(), wl.name
        tol = 1e-5 if wl.dtype == "f32" else 2e-2
        assert rel_l2(y.float().cpu().numpy(), ora) <= tol, wl.name
        assert "spec_mfma" not in names, names
        if wl.dtype == "bf16":
            assert "fused_mfma" in names, names
        if spectral:
            # two algorithms, each within tol of the oracle
            assert rel_l2(y.float().cpu().numpy(), y_ref.float().cpu().numpy()) <= 2 * tol, wl.name
        else:
            assert torch.equal(y, y_ref), wl.name


def test_noalloc_rejects_layers_beyond_its_scratch(sdc):
    # 4096 x 128 channels: 8 MiB of weight fragments against 4 MiB of scratch
    psi = sdc.psi_build(9, 16, 9, 16, (3,), 0.7).to_device()
    x = torch.zeros((1, 4096, 9, 16), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((128, 4096, 3), dtype=torch.bfloat16, device="cuda")
    y = torch.full((1, 128, 9, 16), 7.0, device="cuda")
    with pytest.raises(ValueError, match="scratch"):
        sdc.fused_fwd_noalloc(psi, x, w, y)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())      # nothing was launched
