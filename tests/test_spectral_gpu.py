"""GPU parity of the longitude-spectral fused path (and of the direct matrix-core
path on the same shapes), through the C ABI, against the CPU oracle.

The spectral path evaluates each window's circular correlation along
longitude with real DFTs (the p-shift of the DiscreteContinuousConvS2 page).
Its spectra and the (frequency, (ci, k)) tile are rounded to bf16, so the bar is
the bf16 one: relative L2 <= 2e-2 against the float64 oracle on the same
bf16-rounded inputs.  The shapes below cover every radix of the transform
plans (2, 3, 4, 5), K from 1 to 8, both output-channel tiles, a batch of two,
and isotropic and anisotropic bases.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from disco_workloads import WORKLOADS, Workload, draw_inputs, round_bf16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


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


def worst_band_rel_l2(got, ref, band=32):
    """Largest relative L2 error over bands of `band` consecutive longitude
    frequencies (real DFT along the last axis, full rows on both sides).  The
    spectral path rounds spectra per frequency, so its error is relative in
    every band; an error confined to one of the kernel's 32-frequency items
    shows here even where that band carries little of the output's energy."""
    fg = np.fft.rfft(np.asarray(got, np.float64), axis=-1)
    fr = np.fft.rfft(np.asarray(ref, np.float64), axis=-1)
    worst = 0.0
    for m0 in range(0, fr.shape[-1], band):
        d = np.linalg.norm(fg[..., m0:m0 + band] - fr[..., m0:m0 + band])   # complex norms
        worst = max(worst, float(d / max(np.linalg.norm(fr[..., m0:m0 + band]), 1e-300)))
    return worst


def W(name, B, Ci, Co, nlat, nlon, ks, cut, seed=21):
    return Workload(name, seed, B, Ci, Co, 1, nlat, nlon, nlat, nlon, ks, oracle.num_basis(ks), cut,
                    "bf16")


# nlon / 2 = 60 (4,3,5), 50 (2,5,5), 36 (4,3,3), 30 (2,3,5), 8 (4,2), 40 (2,4,5)
SPECTRAL = [
    W("c4_like", 1, 128, 128, 61, 120, (3, 3), 4 * math.pi / 60),
    W("b2_ci64_co128", 2, 64, 128, 25, 100, (3, 3), 0.45),
    W("iso_k4_co64", 1, 32, 64, 19, 72, (4,), 0.6),
    W("k8_co64", 1, 32, 64, 21, 60, (2, 7), 0.5),
    W("k1_tiny", 1, 32, 64, 9, 16, (1,), 0.7),
    # 41 -> 20 latitudes at 80 longitudes: four output rows gather 8 input
    # rows, the most the spectral kernel takes (equal grids give odd counts)
    Workload("lat_down_8win", 21, 1, 32, 128, 1, 41, 80, 20, 80, (3, 3), oracle.num_basis((3, 3)),
             0.2827, "bf16"),
]


def _prepare(wl):
    x, w = draw_inputs(wl)
    return round_bf16(x), round_bf16(w)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(torch.bfloat16)


def _psi(sdc, wl):
    return sdc.psi_build(wl.nlat_in, wl.nlon_in, wl.nlat_out, wl.nlon_out, wl.kernel_shape,
                         wl.theta_cutoff).to_device()


def _desc(wl):
    return oracle.Desc(wl.nlat_in, wl.nlon_in, wl.nlat_out, wl.nlon_out, wl.kernel_shape,
                       wl.theta_cutoff)


def test_path_selection(sdc, monkeypatch):
    wl = SPECTRAL[0]
    psi = _psi(sdc, wl)
    monkeypatch.setenv("DISCO_FUSED_PATH", "toeplitz")
    assert not sdc.fused_is_spectral(psi, torch.bfloat16, 128, 128, 1)   # direct kernel asked for
    monkeypatch.delenv("DISCO_FUSED_PATH")
    assert sdc.fused_is_spectral(psi, torch.bfloat16, 128, 128, 1)       # the default
    assert sdc.fused_is_spectral(psi, torch.bfloat16, 64, 64, 1)
    assert sdc.fused_is_spectral(psi, torch.float32, 128, 128, 1)        # float32 kernels
    assert not sdc.fused_is_spectral(psi, torch.float32, 128, 256, 1)    # float32: Co <= 128
    assert not sdc.fused_is_spectral(psi, torch.bfloat16, 128, 96, 1)    # Co tile
    assert not sdc.fused_is_spectral(psi, torch.bfloat16, 40, 64, 1)     # 32-channel chunks
    assert not sdc.fused_is_spectral(psi, torch.bfloat16, 128, 128, 2)   # groups
    # stride 2 takes the spectral path only where both transforms have
    # register forms (720 and 1440 input longitudes)
    p2 = sdc.psi_build(33, 64, 17, 32, (3, 3), 4 * math.pi / 16).to_device()
    assert not sdc.fused_is_spectral(p2, torch.bfloat16, 128, 128, 1)
    p3 = sdc.psi_build(31, 720, 16, 360, (3, 3), 4 * math.pi / 30).to_device()
    assert sdc.fused_is_spectral(p3, torch.bfloat16, 64, 64, 1)
    # N / 2 = 7 is not a product of 2, 3 and 5
    p7 = sdc.psi_build(9, 14, 9, 14, (3,), 0.7).to_device()
    assert not sdc.fused_is_spectral(p7, torch.bfloat16, 128, 128, 1)


@pytest.mark.parametrize("path", ["spectral", "toeplitz"])
@pytest.mark.parametrize("wl", SPECTRAL, ids=[w.name for w in SPECTRAL])
def test_fused_paths_small(sdc, wl, path, monkeypatch):
    if path == "toeplitz":
        monkeypatch.setenv("DISCO_FUSED_PATH", "toeplitz")
    else:
        monkeypatch.delenv("DISCO_FUSED_PATH", raising=False)
    _say("fused", path, wl.name)
    x, w = _prepare(wl)
    psi = _psi(sdc, wl)
    assert sdc.fused_is_spectral(psi, torch.bfloat16, wl.Ci, wl.Co, 1) == (path == "spectral")
    bias = np.linspace(-1, 1, wl.Co).astype(np.float32)
    ref = oracle.forward(_desc(wl), x, w, 1)
    refb = oracle.forward(_desc(wl), x, w, 1, bias=bias)
    xd, wd = _dev(x), _dev(w)
    y = sdc.fused_fwd(psi, xd, wd).cpu().numpy()
    err = rel_l2(y, ref)
    _say(f"  rel-L2 {err:.3e}")
    assert err <= TOL_BF16
    if path == "spectral":
        band = worst_band_rel_l2(y, ref)
        _say(f"  worst 32-frequency band rel-L2 {band:.3e}")
        assert band <= TOL_BF16
    bd = torch.from_numpy(bias).cuda()
    for out_dtype in (torch.float32, torch.bfloat16):
        yb = sdc.fused_fwd(psi, xd, wd, bias=bd, out_dtype=out_dtype).float().cpu().numpy()
        assert rel_l2(yb, refb) <= TOL_BF16


def test_spectral_roll_equivariance(sdc, monkeypatch):
    # a longitude shift of x is a phase rotation of its spectrum, which is then
    # rounded to bf16: the rolled output agrees up to that rounding (a wrong
    # shift or index would be off by O(1))
    monkeypatch.delenv("DISCO_FUSED_PATH", raising=False)
    wl = SPECTRAL[1]
    x, w = _prepare(wl)
    psi = _psi(sdc, wl)
    xd, wd = _dev(x), _dev(w)
    y = sdc.fused_fwd(psi, xd, wd).cpu().numpy()
    yr = sdc.fused_fwd(psi, torch.roll(xd, -1, dims=-1).contiguous(), wd).cpu().numpy()
    err = rel_l2(yr, np.roll(y, -1, axis=-1))
    _say(f"spectral roll equivariance rel-L2 {err:.3e}")
    assert err <= 1e-2


def test_spectral_determinism(sdc, monkeypatch):
    monkeypatch.delenv("DISCO_FUSED_PATH", raising=False)
    wl = SPECTRAL[1]
    x, w = _prepare(wl)
    psi = _psi(sdc, wl)
    xd, wd = _dev(x), _dev(w)
    a = sdc.fused_fwd(psi, xd, wd).cpu().numpy()
    b = sdc.fused_fwd(psi, xd, wd).cpu().numpy()
    assert np.array_equal(a, b)


def test_workspace_reuse_across_streams_and_sizes(sdc, monkeypatch):
    """The handle keeps its workspace between calls.  Calls of two batch sizes
    (the workspace grows between them) alternate on two streams without host
    synchronisation; each result must equal, bit for bit, the same call made
    alone on the current stream (the spectral sums run in a fixed order)."""
    monkeypatch.delenv("DISCO_FUSED_PATH", raising=False)
    wl = SPECTRAL[1]   # B = 2
    x, w = _prepare(wl)
    psi = _psi(sdc, wl)
    xd, wd = _dev(x), _dev(w)
    x1 = xd[:1].contiguous()
    assert sdc.fused_is_spectral(psi, torch.bfloat16, wl.Ci, wl.Co, 1)
    want1 = sdc.fused_fwd(psi, x1, wd).cpu().numpy()
    want2 = sdc.fused_fwd(psi, xd, wd).cpu().numpy()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(3):
        y1 = torch.empty((1, wl.Co, wl.nlat_out, wl.nlon_out), device="cuda")
        y2 = torch.empty((2, wl.Co, wl.nlat_out, wl.nlon_out), device="cuda")
        for t in (y1, y2):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        sdc.fused_fwd(psi, x1, wd, y=y1, stream=s1)
        sdc.fused_fwd(psi, xd, wd, y=y2, stream=s2)
        outs.append((y1, y2))
    torch.cuda.synchronize()
    for rep, (y1, y2) in enumerate(outs):
        _say(f"workspace reuse rep {rep}")
        assert np.array_equal(y1.cpu().numpy(), want1)
        assert np.array_equal(y2.cpu().numpy(), want2)
    # and against the oracle, once
    ref = oracle.forward(_desc(wl), x, w, 1)
    assert rel_l2(outs[-1][1].cpu().numpy(), ref) <= TOL_BF16


def _sample_rows(nlat):
    rows = {0, 1, 2, 5, nlat // 7, nlat // 3, nlat // 2, (2 * nlat) // 3, nlat - 6, nlat - 2, nlat - 1}
    return sorted(r for r in rows if 0 <= r < nlat)


def _sample_cols(nlon, seed=0):
    rng = np.random.default_rng(seed)
    cols = {0, 1, nlon - 1, nlon // 2} | set(rng.choice(nlon, size=min(nlon, 28), replace=False).tolist())
    return sorted(cols)


@pytest.mark.parametrize("path", ["spectral", "toeplitz"])
def test_full_size_c4_paths(sdc, path, monkeypatch):
    """721x1440, 128 -> 128 channels, K = 7, bf16: both fused algorithms (the
    benchmark times the spectral one, the default)."""
    if path == "toeplitz":
        monkeypatch.setenv("DISCO_FUSED_PATH", "toeplitz")
    else:
        monkeypatch.delenv("DISCO_FUSED_PATH", raising=False)
    wl = WORKLOADS["c4"]
    _say("full size c4", path)
    x, w = _prepare(wl)
    psi = _psi(sdc, wl)
    assert sdc.fused_is_spectral(psi, torch.bfloat16, wl.Ci, wl.Co, 1) == (path == "spectral")
    y = sdc.fused_fwd(psi, _dev(x), _dev(w))
    torch.cuda.synchronize()
    rows, cols = _sample_rows(wl.nlat_out), _sample_cols(wl.nlon_out)
    ref = oracle.forward(_desc(wl), x, w, 1, rows=rows, cols_out=cols)
    got = y[:, :, rows][:, :, :, cols].cpu().numpy()
    err = rel_l2(got, ref)
    _say(f"  c4 {path} rel-L2 {err:.3e}")
    assert err <= TOL_BF16
    if path == "spectral":
        # whole rows (all 1440 longitudes) at a near-polar, a mid and the
        # equatorial latitude: error per band of 32 frequencies
        frows = [30, 200, 360]
        fref = oracle.forward(_desc(wl), x, w, 1, rows=frows)
        band = worst_band_rel_l2(y[:, :, frows].cpu().numpy(), fref)
        _say(f"  c4 spectral worst 32-frequency band rel-L2 {band:.3e}")
        assert band <= TOL_BF16


# half lengths with register-resident transforms: 720 = 16 x 45 (0.25 degree
# grids), 360 = 8 x 45, 180 = 4 x 45; outputs compared at sampled longitudes
REG = [
    W("n1440", 1, 32, 64, 13, 1440, (3, 3), 0.5),
    W("n720_b2", 2, 32, 128, 11, 720, (3,), 0.6),
    W("n360", 1, 64, 64, 19, 360, (2, 2), 0.4),
]


@pytest.mark.parametrize("wl", REG, ids=[w.name for w in REG])
def test_register_transforms(sdc, wl, monkeypatch):
    monkeypatch.delenv("DISCO_FUSED_PATH", raising=False)
    _say("register transforms", wl.name)
    x, w = _prepare(wl)
    psi = _psi(sdc, wl)
    assert sdc.fused_is_spectral(psi, torch.bfloat16, wl.Ci, wl.Co, 1)
    cols = _sample_cols(wl.nlon_out, seed=3)
    bias = np.linspace(-1, 1, wl.Co).astype(np.float32)
    ref = oracle.forward(_desc(wl), x, w, 1, cols_out=cols)
    refb = oracle.forward(_desc(wl), x, w, 1, cols_out=cols, bias=bias)
    xd, wd = _dev(x), _dev(w)
    y = sdc.fused_fwd(psi, xd, wd)[..., cols].cpu().numpy()
    err = rel_l2(y, ref)
    _say(f"  rel-L2 {err:.3e}")
    assert err <= TOL_BF16
    bd = torch.from_numpy(bias).cuda()
    for out_dtype in (torch.float32, torch.bfloat16):
        yb = sdc.fused_fwd(psi, xd, wd, bias=bd, out_dtype=out_dtype)[..., cols].float().cpu().numpy()
        assert rel_l2(yb, refb) <= TOL_BF16


# longitude stride 2: the stride-1 correlation's spectrum folded onto the
# output grid's frequencies before the inverse transform; 15 input rows per
# output row (two window-sum MFMA steps), like the 361x720 -> 181x360 layer
STRIDE2 = [
    Workload("s2_720_co64", 23, 1, 64, 64, 1, 61, 720, 31, 360, (3, 3), oracle.num_basis((3, 3)),
             4 * math.pi / 30, "bf16"),
    Workload("s2_1440_co128_b2", 24, 2, 32, 128, 1, 25, 1440, 13, 720, (3,), 3, 4 * math.pi / 12,
             "bf16"),
]


@pytest.mark.parametrize("path", ["spectral", "spectral16", "toeplitz"])
@pytest.mark.parametrize("wl", STRIDE2, ids=[w.name for w in STRIDE2])
def test_stride2_spectral(sdc, wl, path, monkeypatch):
    """spectral: rows of up to 15 windows in two halves on the 8-window
    kernel; spectral16: the same rows on the 16-window kernel
    (DISCO_SPEC_HALVES=0); toeplitz: the direct matrix-core kernel."""
    monkeypatch.delenv("DISCO_SPEC_HALVES", raising=False)
    if path == "toeplitz":
        monkeypatch.setenv("DISCO_FUSED_PATH", "toeplitz")
    else:
        monkeypatch.delenv("DISCO_FUSED_PATH", raising=False)
        if path == "spectral16":
            monkeypatch.setenv("DISCO_SPEC_HALVES", "0")
        sdc.kernel_timing(True)
    _say("stride 2", path, wl.name)
    x, w = _prepare(wl)
    psi = _psi(sdc, wl)
    assert sdc.fused_is_spectral(psi, torch.bfloat16, wl.Ci, wl.Co, 1) == (path != "toeplitz")
    xd, wd = _dev(x), _dev(w)
    bias = np.linspace(-1, 1, wl.Co).astype(np.float32)
    try:
        y = sdc.fused_fwd(psi, xd, wd, bias=torch.from_numpy(bias).cuda()).cpu().numpy()
    finally:
        ran = set(sdc.kernel_timing_read())
        sdc.kernel_timing(False)
    if path != "toeplitz":
        assert "spec_mfma" in ran, ran
    cols = _sample_cols(wl.nlon_out, seed=5)
    ref = oracle.forward(_desc(wl), x, w, 1, cols_out=cols, bias=bias)
    err = rel_l2(y[..., cols], ref)
    _say(f"  rel-L2 {err:.3e}")
    assert err <= TOL_BF16
    if path != "toeplitz":
        frows = [0, wl.nlat_out // 3, wl.nlat_out // 2]
        fref = oracle.forward(_desc(wl), x, w, 1, rows=frows)
        band = worst_band_rel_l2(y[:, :, frows] - bias[None, :, None, None], fref)
        _say(f"  worst 32-frequency band rel-L2 {band:.3e}")
        assert band <= TOL_BF16


# float32 layers at stride 1: float32 spectra and Psi_hat, both sums on the
# vector ALUs in float32; held to the float32 bar
SPEC32 = [
    Workload("f32_c2_like", 25, 2, 32, 32, 1, 33, 64, 33, 64, (3, 3), 7, 4 * math.pi / 32, "f32"),
    Workload("f32_ragged", 26, 1, 5, 7, 1, 17, 32, 17, 32, (3,), 3, 0.5, "f32"),
    Workload("f32_co128_ci40_k8", 27, 1, 40, 128, 1, 25, 48, 25, 48, (2, 7), 8, 0.5, "f32"),
    Workload("f32_wide_cap", 28, 1, 3, 2, 1, 17, 32, 17, 32, (3, 3), 7, 2.5, "f32"),
    Workload("f32_k1", 29, 1, 2, 2, 1, 9, 16, 9, 16, (1,), 1, 0.7, "f32"),
]


@pytest.mark.parametrize("wl", SPEC32, ids=[w.name for w in SPEC32])
def test_float32_spectral(sdc, wl, monkeypatch):
    monkeypatch.delenv("DISCO_FUSED_PATH", raising=False)
    _say("float32 spectral", wl.name)
    x, w = draw_inputs(wl)
    psi = _psi(sdc, wl)
    assert sdc.fused_is_spectral(psi, torch.float32, wl.Ci, wl.Co, 1)
    xd, wd = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
    sdc.kernel_timing(True)
    try:
        y = sdc.fused_fwd(psi, xd, wd).cpu().numpy()
        names = set(sdc.kernel_timing_read())
    finally:
        sdc.kernel_timing(False)
    assert "spec32_conv" in names, names
    ref = oracle.forward(_desc(wl), x, w, 1)
    err, band = rel_l2(y, ref), worst_band_rel_l2(y, ref)
    _say(f"  rel-L2 {err:.3e}, worst 32-frequency band {band:.3e}")
    assert err <= 1e-5
    assert band <= 1e-4
    bias = np.linspace(-1, 1, wl.Co).astype(np.float32)
    refb = oracle.forward(_desc(wl), x, w, 1, bias=bias)
    yb = sdc.fused_fwd(psi, xd, wd, bias=torch.from_numpy(bias).cuda()).cpu().numpy()
    assert rel_l2(yb, refb) <= 1e-5
    yh = sdc.fused_fwd(psi, xd, wd, bias=torch.from_numpy(bias).cuda(),
                       out_dtype=torch.bfloat16).float().cpu().numpy()
    assert rel_l2(yh, refb) <= 8e-3
    # the direct kernel on the same layer agrees to float32 rounding
    monkeypatch.setenv("DISCO_FUSED_PATH", "toeplitz")
    assert not sdc.fused_is_spectral(psi, torch.float32, wl.Ci, wl.Co, 1)
    yd = sdc.fused_fwd(psi, xd, wd).cpu().numpy()
    assert rel_l2(yd, y) <= 2e-6


@pytest.mark.parametrize("case", ["stockham", "register"])
def test_kernel_timing_names_the_spectral_kernels(sdc, case, monkeypatch):
    """The launches of one call: with the Stockham transforms (100
    longitudes) the weight fragments take a launch of their own; the register
    transforms' launch (720 longitudes) writes them itself."""
    monkeypatch.delenv("DISCO_FUSED_PATH", raising=False)
    wl = SPECTRAL[1] if case == "stockham" else REG[1]
    x, w = _prepare(wl)
    psi = _psi(sdc, wl)
    xd, wd = _dev(x), _dev(w)
    sdc.fused_fwd(psi, xd, wd)            # not recorded
    sdc.kernel_timing(True)
    try:
        for _ in range(3):
            sdc.fused_fwd(psi, xd, wd)
        t = sdc.kernel_timing_read()
    finally:
        sdc.kernel_timing(False)
    _say("kernel timing", t)
    want = ["spec_rfft", "spec_mfma", "spec_irfft"]
    assert list(t) == (["spec_prep_w"] + want if case == "stockham" else want)
    for name, (ms, n) in t.items():
        assert n == 3 and ms > 0.0, name
    sdc.fused_fwd(psi, xd, wd)            # timing off again: nothing recorded
    torch.cuda.synchronize()
    assert sdc.kernel_timing_read() == {}
