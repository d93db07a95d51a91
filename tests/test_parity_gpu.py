"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every comparison uses the same seeded inputs on both sides; bf16 cases feed
the oracle the bf16-rounded values.  Bar: relative L2 error over the compared
outputs <= 1e-5 for float32 and <= 2e-2 for bf16 inputs with float32
accumulation.  Reduced grids are compared on every output; the full-size
benchmark cases are compared on sampled output rows and longitudes (all
batches and channels), in the same launch configuration the benchmark times.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from disco_workloads import WORKLOADS, Workload, draw_inputs, round_bf16, small_variant

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


def max_rel_l2_slices(a, b):
    """Largest relative L2 error over single output channels (axis 1) and over
    single output rows (axis 2) of [B, C, rows, cols] arrays: an error confined
    to one channel or one row shows here even when the global figure hides it."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    worst = 0.0
    for axis in (1, 2):
        for i in range(a.shape[axis]):
            worst = max(worst, rel_l2(np.take(a, i, axis=axis), np.take(b, i, axis=axis)))
    return worst


def _tdtype(dt):
    return torch.float32 if dt == "f32" else torch.bfloat16


def _prepare(wl, seed=None):
    x, w = draw_inputs(wl, seed)
    if wl.dtype == "bf16":
        x, w = round_bf16(x), round_bf16(w)
    return x, w


def _to_dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(_tdtype(dt))


def _desc(wl):
    return oracle.Desc(wl.nlat_in, wl.nlon_in, wl.nlat_out, wl.nlon_out, wl.kernel_shape,
                       wl.theta_cutoff)


def _psi(sdc, wl):
    return sdc.psi_build(wl.nlat_in, wl.nlon_in, wl.nlat_out, wl.nlon_out, wl.kernel_shape,
                         wl.theta_cutoff).to_device()


def W(name, B, Ci, Co, G, nli, nfi, nlo, nfo, ks, cut, dt, seed=11):
    return Workload(name, seed, B, Ci, Co, G, nli, nfi, nlo, nfo, ks, oracle.num_basis(ks), cut,
                    dt)


SMALL = [
    W("iso_f32", 2, 3, 5, 1, 17, 32, 17, 32, (3,), 0.5, "f32"),
    W("aniso_f32_s2", 1, 4, 4, 1, 33, 64, 17, 32, (3, 3), 4 * math.pi / 16, "f32"),
    W("aniso_f32_s4_ragged", 2, 5, 3, 1, 25, 100, 13, 25, (3, 3), 0.45, "f32"),
    W("groups_f32", 1, 6, 4, 2, 33, 64, 33, 64, (3, 3), 4 * math.pi / 32, "f32"),
    W("depthwise_f32", 1, 8, 8, 8, 33, 64, 17, 32, (5, 4), 6 * math.pi / 16, "f32"),
    W("multiplier_f32", 1, 3, 6, 3, 17, 32, 17, 32, (2, 2), 0.6, "f32"),
    W("iso_bf16", 1, 32, 32, 1, 33, 64, 33, 64, (3,), 4 * math.pi / 32, "bf16"),
    W("aniso_bf16", 2, 64, 64, 1, 49, 96, 49, 96, (3, 3), 4 * math.pi / 48, "bf16"),
    W("aniso_bf16_s2", 1, 64, 48, 1, 73, 144, 37, 72, (3, 3), 4 * math.pi / 36, "bf16"),
    W("c4_like_bf16", 1, 128, 128, 1, 61, 120, 61, 120, (3, 3), 4 * math.pi / 60, "bf16"),
    W("odd_bf16", 1, 40, 24, 2, 21, 40, 21, 40, (3, 3), 0.5, "bf16"),
    W("k1_f32", 1, 2, 2, 1, 9, 16, 9, 16, (1,), 0.7, "f32"),
    W("nlat2_f32", 1, 2, 3, 1, 2, 8, 2, 4, (2,), 1.0, "f32"),
    W("wide_cap_f32", 1, 2, 2, 1, 17, 32, 17, 32, (3, 3), 2.5, "f32"),
    # the register-tiled depthwise kernel (four outputs per thread, 64 to 256
    # threads): one pass of 192 threads at stride 1, one of 128 at stride 2,
    # two passes of 256 at strides 1 and 2 (rows longer than 1024 outputs,
    # with polar windows spanning the whole ring), a multiplier of 2 and bf16
    W("depthwise_long_s1_f32", 1, 4, 4, 4, 13, 600, 13, 600, (3, 3), 0.5, "f32"),
    W("depthwise_long_s2_f32", 2, 3, 3, 3, 17, 1024, 9, 512, (4,), 0.6, "f32"),
    W("depthwise_2pass_s1_f32", 1, 2, 2, 2, 9, 1440, 9, 1440, (3,), 0.6, "f32"),
    W("depthwise_2pass_s2_f32", 1, 2, 4, 2, 9, 2400, 5, 1200, (2, 2), 0.9, "f32"),
    W("depthwise_s2_bf16", 1, 5, 5, 5, 25, 96, 13, 48, (5, 4), 0.5, "bf16"),
    # grouped bf16 layers on the matrix-core einsum: 64 output channels per
    # group (the streamed kernel) and 48 per group (the general tiled kernel)
    W("grouped_stream_bf16", 1, 64, 128, 2, 33, 64, 33, 64, (3, 3), 4 * math.pi / 32, "bf16"),
    W("grouped_general_bf16", 2, 64, 96, 2, 33, 64, 17, 32, (3, 3), 4 * math.pi / 16, "bf16"),
]

# which einsum kernel each grouped bf16 case must run (the dispatch rule of the
# C ABI: bf16 groups of 64 or 128 output channels with (Ci/G) K a multiple of
# 32 stream, other bf16 groups of >= 32 output channels use the tiled kernel)
EINSUM_KERNEL = {"grouped_stream_bf16": "einsum_stream_bf16",
                 "grouped_general_bf16": "einsum_mfma_bf16"}


def kernels_run(sdc, fn):
    """Run fn() with the library's per-kernel timing on; return (result,
    names of the kernels it launched)."""
    sdc.kernel_timing(True)
    try:
        out = fn()
        names = set(sdc.kernel_timing_read())
    finally:
        sdc.kernel_timing(False)
    return out, names


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_contract_small(sdc, wl):
    _say("contract", wl.name)
    x, _ = _prepare(wl)
    d = _desc(wl)
    psi = _psi(sdc, wl)
    xk = sdc.contract(psi, _to_dev(x, wl.dtype)).float().cpu().numpy()
    torch.cuda.synchronize()
    ref = oracle.contract(d, x)
    assert rel_l2(xk, ref) <= TOL[wl.dtype]
    if wl.dtype == "f32":
        xk32 = sdc.contract(psi, _to_dev(x, "f32"), xk_dtype=torch.float32).cpu().numpy()
        assert rel_l2(xk32, ref) <= 1e-5


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_einsum_small(sdc, wl):
    _say("einsum", wl.name)
    rng = np.random.default_rng(5)
    xk = rng.standard_normal((wl.B, wl.Ci, wl.K, wl.nlat_out, wl.nlon_out)).astype(np.float32)
    _, w = _prepare(wl)
    if wl.dtype == "bf16":
        xk = round_bf16(xk)
    ref = oracle.einsum(xk, w, wl.groups)
    xkd, wd = _to_dev(xk, wl.dtype), _to_dev(w, wl.dtype)
    y, names = kernels_run(sdc, lambda: sdc.einsum(xkd, wd, groups=wl.groups).cpu().numpy())
    if wl.name in EINSUM_KERNEL:
        assert EINSUM_KERNEL[wl.name] in names, names
    # inputs are exact on both sides: only float32 accumulation order differs
    assert rel_l2(y, ref) <= (1e-5 if wl.dtype == "f32" else 1e-5 * 10)
    assert max_rel_l2_slices(y, ref) <= (1e-5 if wl.dtype == "f32" else 1e-4)


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_fused_and_unfused_small(sdc, wl):
    _say("fused", wl.name)
    x, w = _prepare(wl)
    d = _desc(wl)
    ref = oracle.forward(d, x, w, wl.groups)
    psi = _psi(sdc, wl)
    xd, wd = _to_dev(x, wl.dtype), _to_dev(w, wl.dtype)
    yf = sdc.fused_fwd(psi, xd, wd, groups=wl.groups).cpu().numpy()
    assert rel_l2(yf, ref) <= TOL[wl.dtype], "fused"
    assert max_rel_l2_slices(yf, ref) <= TOL[wl.dtype], "fused, per channel / row"
    yu, names = kernels_run(sdc, lambda: sdc.einsum(sdc.contract(psi, xd), wd,
                                                    groups=wl.groups).cpu().numpy())
    if wl.name in EINSUM_KERNEL:
        assert EINSUM_KERNEL[wl.name] in names, names
    assert rel_l2(yu, ref) <= TOL[wl.dtype], "unfused"
    assert max_rel_l2_slices(yu, ref) <= TOL[wl.dtype], "unfused, per channel / row"


def test_bias_and_bf16_output(sdc):
    wl = SMALL[8]
    x, w = _prepare(wl)
    bias = np.linspace(-1, 1, wl.Co).astype(np.float32)
    ref = oracle.forward(_desc(wl), x, w, wl.groups, bias=bias)
    psi = _psi(sdc, wl)
    xd, wd = _to_dev(x, wl.dtype), _to_dev(w, wl.dtype)
    bd = torch.from_numpy(bias).cuda()
    for out_dtype in (torch.float32, torch.bfloat16):
        yf = sdc.fused_fwd(psi, xd, wd, bias=bd, out_dtype=out_dtype).float().cpu().numpy()
        assert rel_l2(yf, ref) <= TOL["bf16"]
        yu = sdc.einsum(sdc.contract(psi, xd), wd, bias=bd, out_dtype=out_dtype).float().cpu().numpy()
        assert rel_l2(yu, ref) <= TOL["bf16"]
    wl = SMALL[3]
    x, w = _prepare(wl)
    bias = np.linspace(-1, 1, wl.Co).astype(np.float32)
    ref = oracle.forward(_desc(wl), x, w, wl.groups, bias=bias)
    psi = _psi(sdc, wl)
    yf = sdc.fused_fwd(psi, _to_dev(x, "f32"), _to_dev(w, "f32"), groups=wl.groups,
                       bias=torch.from_numpy(bias).cuda()).cpu().numpy()
    assert rel_l2(yf, ref) <= 1e-5


def test_empty_batch_is_noop(sdc):
    wl = SMALL[0]
    psi = _psi(sdc, wl)
    x = torch.zeros((0, wl.Ci, wl.nlat_in, wl.nlon_in), device="cuda")
    w = torch.zeros((wl.Co, wl.Ci, wl.K), device="cuda")
    y = sdc.fused_fwd(psi, x, w)
    assert y.shape[0] == 0
    xk = sdc.contract(psi, x)
    assert xk.shape[0] == 0


def test_device_argument_errors(sdc):
    wl = SMALL[0]
    psi = _psi(sdc, wl)
    x = torch.zeros((1, wl.Ci, wl.nlat_in, wl.nlon_in))           # host tensor
    w = torch.zeros((wl.Co, wl.Ci, wl.K), device="cuda")
    with pytest.raises(ValueError):
        sdc.fused_fwd(psi, x, w)
    xd = x.cuda()
    with pytest.raises(ValueError):
        sdc.fused_fwd(psi, xd, torch.zeros((wl.Co, wl.Ci, wl.K + 1), device="cuda"))
    # output aliasing an input
    y = torch.zeros((1, wl.Co, wl.nlat_out, wl.nlon_out), device="cuda")
    big = torch.zeros(max(xd.numel(), y.numel()), device="cuda")
    with pytest.raises(ValueError):
        sdc.fused_fwd(psi, big[:xd.numel()].view_as(xd), w, y=big[:y.numel()].view_as(y))
    # unuploaded handle
    p2 = sdc.psi_build(wl.nlat_in, wl.nlon_in, wl.nlat_out, wl.nlon_out, wl.kernel_shape,
                       wl.theta_cutoff)
    with pytest.raises(ValueError):
        sdc.fused_fwd(p2, xd, w)


@pytest.mark.parametrize("which", ["aniso_f32_s2", "aniso_bf16_s2", "c4_like_bf16", "depthwise_f32"])
def test_roll_equivariance_gpu(sdc, which):
    wl = [w for w in SMALL if w.name == which][0]
    x, w = _prepare(wl)
    psi = _psi(sdc, wl)
    s = wl.nlon_in // wl.nlon_out
    xd, wd = _to_dev(x, wl.dtype), _to_dev(w, wl.dtype)
    y = sdc.fused_fwd(psi, xd, wd, groups=wl.groups).cpu().numpy()
    yr = sdc.fused_fwd(psi, torch.roll(xd, -s, dims=-1).contiguous(), wd,
                       groups=wl.groups).cpu().numpy()
    diff = np.max(np.abs(yr - np.roll(y, -1, axis=-1)))
    _say(f"roll equivariance {which}: max |diff| = {diff:.3e}")
    if wl.dtype == "f32":
        # vector-ALU paths sum every output in the same order: exact
        assert diff == 0.0
    elif sdc.fused_is_spectral(psi, torch.bfloat16, wl.Ci, wl.Co, wl.groups):
        # longitude-spectral path: the shift is a phase rotation of the input
        # spectrum, which is rounded to bf16, so equal up to that rounding
        assert rel_l2(yr, np.roll(y, -1, axis=-1)) <= 1e-2
    else:
        # the matrix-core path sums within MFMA tiles in an order that depends
        # on the output's position in its 4-output block, and then rounds the
        # K-expanded tile to bf16: equal up to rounding
        assert rel_l2(yr, np.roll(y, -1, axis=-1)) <= 1e-4


def test_determinism(sdc):
    wl = SMALL[9]
    x, w = _prepare(wl)
    psi = _psi(sdc, wl)
    xd, wd = _to_dev(x, wl.dtype), _to_dev(w, wl.dtype)
    a = sdc.fused_fwd(psi, xd, wd).cpu().numpy()
    b = sdc.fused_fwd(psi, xd, wd).cpu().numpy()
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# full-size benchmark cases
# ---------------------------------------------------------------------------
def _sample_rows(nlat):
    rows = {0, 1, 2, 5, nlat // 7, nlat // 3, nlat // 2, (2 * nlat) // 3, nlat - 6, nlat - 2, nlat - 1}
    return sorted(r for r in rows if 0 <= r < nlat)


def _sample_cols(nlon, seed=0):
    rng = np.random.default_rng(seed)
    cols = {0, 1, nlon - 1, nlon // 2} | set(rng.choice(nlon, size=min(nlon, 28), replace=False).tolist())
    return sorted(cols)


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4", "c5"])
def test_full_size_fused(sdc, key):
    wl = WORKLOADS[key]
    _say("full size fused", key)
    x, w = _prepare(wl)
    d = _desc(wl)
    psi = _psi(sdc, wl)
    xd, wd = _to_dev(x, wl.dtype), _to_dev(w, wl.dtype)
    y = sdc.fused_fwd(psi, xd, wd, groups=wl.groups)
    torch.cuda.synchronize()
    if key == "c1":
        rows, cols = list(range(wl.nlat_out)), list(range(wl.nlon_out))
    elif key == "c2":
        rows, cols = list(range(wl.nlat_out)), _sample_cols(wl.nlon_out)
    else:
        rows, cols = _sample_rows(wl.nlat_out), _sample_cols(wl.nlon_out)
    ref = oracle.forward(d, x, w, wl.groups, rows=rows, cols_out=cols)
    got = y[:, :, rows][:, :, :, cols].cpu().numpy()
    err = rel_l2(got, ref)
    worst = max_rel_l2_slices(got, ref)
    _say(f"{key} fused rel-L2 {err:.3e}, worst channel/row {worst:.3e}")
    assert err <= TOL[wl.dtype]
    assert worst <= TOL[wl.dtype]


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4", "c5"])
def test_full_size_unfused(sdc, key):
    wl = WORKLOADS[key]
    _say("full size unfused", key)
    x, w = _prepare(wl)
    d = _desc(wl)
    psi = _psi(sdc, wl)
    xd, wd = _to_dev(x, wl.dtype), _to_dev(w, wl.dtype)
    xk = sdc.contract(psi, xd)
    y = sdc.einsum(xk, wd, groups=wl.groups)
    torch.cuda.synchronize()
    if key == "c1":
        rows, cols = list(range(wl.nlat_out)), list(range(wl.nlon_out))
    elif key == "c2":
        rows, cols = list(range(wl.nlat_out)), _sample_cols(wl.nlon_out, 1)
    else:
        rows, cols = _sample_rows(wl.nlat_out), _sample_cols(wl.nlon_out, 1)
    xk_ref = oracle.contract(d, x, rows=rows, cols_out=cols)
    ref = oracle.einsum(xk_ref, w, wl.groups)
    got_xk = xk[:, :, :, rows][:, :, :, :, cols].float().cpu().numpy()
    got = y[:, :, rows][:, :, :, cols].cpu().numpy()
    e1, e2 = rel_l2(got_xk, xk_ref), rel_l2(got, ref)
    worst = max_rel_l2_slices(got, ref)
    _say(f"{key} unfused rel-L2 xk {e1:.3e} y {e2:.3e}, worst channel/row {worst:.3e}")
    assert e1 <= TOL[wl.dtype]
    assert e2 <= TOL[wl.dtype]
    assert worst <= TOL[wl.dtype]


# the generic fused kernel at 721x1440: polar windows span the whole ring of
# 1440 longitudes, so its staged samples come in bounded tap chunks
WIDE = [
    W("wide_f32_c32", 1, 32, 32, 1, 721, 1440, 721, 1440, (3, 3), 4 * math.pi / 720, "f32"),
    W("wide_bf16_g2", 1, 64, 64, 2, 721, 1440, 721, 1440, (3, 3), 4 * math.pi / 720, "bf16"),
]


@pytest.mark.parametrize("wl", WIDE, ids=[w.name for w in WIDE])
def test_fused_generic_full_ring_windows(sdc, wl, monkeypatch):
    # the direct kernels (float32 stride-1 layers otherwise go spectral)
    monkeypatch.setenv("DISCO_FUSED_PATH", "toeplitz")
    _say("generic fused, full-ring windows", wl.name)
    x, w = _prepare(wl)
    psi = _psi(sdc, wl)
    xd, wd = _to_dev(x, wl.dtype), _to_dev(w, wl.dtype)
    y, names = kernels_run(sdc, lambda: sdc.fused_fwd(psi, xd, wd, groups=wl.groups))
    assert "fused_generic" in names, names
    rows, cols = _sample_rows(wl.nlat_out), _sample_cols(wl.nlon_out, 2)
    ref = oracle.forward(_desc(wl), x, w, wl.groups, rows=rows, cols_out=cols)
    got = y[:, :, rows][:, :, :, cols].cpu().numpy()
    err, worst = rel_l2(got, ref), max_rel_l2_slices(got, ref)
    _say(f"  rel-L2 {err:.3e}, worst channel/row {worst:.3e}")
    assert err <= TOL[wl.dtype]
    assert worst <= TOL[wl.dtype]
