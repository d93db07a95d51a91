"""GPU parity of the gradients (the adjoints of the forward equation's two
linear maps on the DiscreteContinuousConvS2 page; its fused mode recomputes
X_K in the backward pass) through the C ABI, against the CPU oracle's
`contract_transpose`, `einsum_grad_xk`, `einsum_grad_w` and `backward`.

All gradient sums run in float32 on the GPU and in float64 in the oracle, on
the same inputs (bf16 inputs are exact bf16 values on both sides), so every
case is held to relative L2 <= 1e-5 (<= 2e-5 where bf16 outputs are not
involved is not needed: the float32 bar applies throughout).  Cases cover
strides 1, 2 and 4, ragged sizes, groups, depthwise and channel-multiplier
layers, K = 1, an nphi = 3 basis (not mirror-symmetric, so a flipped shift
sign fails), slabs of the fused backward (a layer large enough for several),
full-ring polar windows, an empty batch, and the full-size 721x1440 layer on
channel subsets.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from disco_workloads import WORKLOADS, Workload, draw_inputs, round_bf16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-5


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


def W(name, B, Ci, Co, G, nli, nfi, nlo, nfo, ks, cut, dt, seed=31):
    return Workload(name, seed, B, Ci, Co, G, nli, nfi, nlo, nfo, ks, oracle.num_basis(ks), cut,
                    dt)


CASES = [
    W("iso_f32", 2, 3, 5, 1, 17, 32, 17, 32, (3,), 0.5, "f32"),
    W("aniso_nphi3_f32", 1, 4, 3, 1, 25, 48, 25, 48, (3, 3), 0.45, "f32"),
    W("s2_groups_f32", 2, 6, 4, 2, 33, 64, 17, 32, (3, 3), 4 * math.pi / 16, "f32"),
    W("s4_ragged_f32", 1, 5, 3, 1, 25, 100, 13, 25, (3, 3), 0.45, "f32"),
    W("depthwise_f32", 1, 8, 8, 8, 33, 64, 17, 32, (5, 4), 6 * math.pi / 16, "f32"),
    W("multiplier_f32", 1, 3, 6, 3, 17, 32, 17, 32, (2, 2), 0.6, "f32"),
    W("k1_f32", 1, 2, 2, 1, 9, 16, 9, 16, (1,), 0.7, "f32"),
    W("c4_like_bf16", 1, 64, 64, 1, 61, 120, 61, 120, (3, 3), 4 * math.pi / 60, "bf16"),
    W("s2_bf16", 1, 32, 16, 1, 73, 144, 37, 72, (3, 3), 4 * math.pi / 36, "bf16"),
    # one input channel per group in bf16 (the folded grad_x and the X_K-free
    # grad_w on bf16 operands)
    W("depthwise_bf16", 1, 8, 8, 8, 33, 64, 17, 32, (5, 4), 6 * math.pi / 16, "bf16"),
    # 2304 longitudes at stride 1: the register-tiled grad_x takes two items
    # per thread, and polar windows span the whole ring
    W("depthwise_wide_s1_f32", 1, 2, 2, 2, 9, 2304, 9, 2304, (3,), 0.5, "f32"),
]


def _inputs(wl, seed=7):
    x, w = draw_inputs(wl)
    if wl.dtype == "bf16":
        x, w = round_bf16(x), round_bf16(w)
    rng = np.random.default_rng(seed)
    gy = rng.standard_normal((wl.B, wl.Co, wl.nlat_out, wl.nlon_out)).astype(np.float32)
    return x, w, gy


def _dev(a, dt):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.to(torch.float32 if dt == "f32" else torch.bfloat16)


def _desc(wl):
    return oracle.Desc(wl.nlat_in, wl.nlon_in, wl.nlat_out, wl.nlon_out, wl.kernel_shape,
                       wl.theta_cutoff)


def _psi(sdc, wl):
    return sdc.psi_build(wl.nlat_in, wl.nlon_in, wl.nlat_out, wl.nlon_out, wl.kernel_shape,
                         wl.theta_cutoff).to_device()


@pytest.mark.parametrize("wl", CASES, ids=[c.name for c in CASES])
def test_contract_transpose(sdc, wl):
    _say("contract_transpose", wl.name)
    d = _desc(wl)
    csr = oracle.psi(d)
    rng = np.random.default_rng(3)
    gxk = rng.standard_normal((wl.B, wl.Ci, wl.K, wl.nlat_out, wl.nlon_out)).astype(np.float32)
    if wl.dtype == "bf16":
        gxk = round_bf16(gxk)
    ref = oracle.contract_transpose(d, gxk, csr=csr)
    psi = _psi(sdc, wl)
    gx = sdc.contract_transpose(psi, _dev(gxk, wl.dtype)).cpu().numpy()
    err = rel_l2(gx, ref)
    _say(f"  rel-L2 {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("wl", CASES, ids=[c.name for c in CASES])
def test_einsum_grads(sdc, wl):
    _say("einsum grads", wl.name)
    x, w, gy = _inputs(wl)
    rng = np.random.default_rng(4)
    xk = rng.standard_normal((wl.B, wl.Ci, wl.K, wl.nlat_out, wl.nlon_out)).astype(np.float32)
    if wl.dtype == "bf16":
        xk = round_bf16(xk)
    gyd = torch.from_numpy(gy).cuda()
    gw = sdc.einsum_grad_w(_dev(xk, wl.dtype), gyd, groups=wl.groups).cpu().numpy()
    gw_ref = oracle.einsum_grad_w(gy, xk, wl.groups)
    assert rel_l2(gw, gw_ref) <= TOL, "grad_w"
    gxk = sdc.einsum_grad_xk(gyd, _dev(w, wl.dtype), groups=wl.groups).cpu().numpy()
    gxk_ref = oracle.einsum_grad_xk(gy, w, wl.groups)
    assert rel_l2(gxk, gxk_ref) <= TOL, "grad_xk"
    # bf16 gradient input and output: one rounding of the output
    gxk16 = sdc.einsum_grad_xk(gyd.to(torch.bfloat16), _dev(w, wl.dtype), groups=wl.groups,
                               out_dtype=torch.bfloat16).float().cpu().numpy()
    ref16 = oracle.einsum_grad_xk(round_bf16(gy), w, wl.groups)
    assert rel_l2(gxk16, ref16) <= 8e-3, "grad_xk bf16"


@pytest.mark.parametrize("wl", [CASES[7], CASES[8]], ids=[CASES[7].name, CASES[8].name])
def test_einsum_grad_w_matrix_cores(sdc, wl):
    """einsum_grad_w with a bf16 gradient on the matrix cores (split-K over
    points), the saved X_K in bf16 and in float32, against the oracle."""
    _say("grad_w on matrix cores", wl.name)
    x, w, gy = _inputs(wl)
    gy = round_bf16(gy)
    rng = np.random.default_rng(4)
    xk = round_bf16(rng.standard_normal((wl.B, wl.Ci, wl.K, wl.nlat_out, wl.nlon_out))
                    .astype(np.float32))
    ref = oracle.einsum_grad_w(gy, xk, wl.groups)
    for xdt in ("bf16", "f32"):
        sdc.kernel_timing(True)
        try:
            gw = sdc.einsum_grad_w(_dev(xk, xdt), _dev(gy, "bf16"), groups=wl.groups).cpu().numpy()
            ran = set(sdc.kernel_timing_read())
        finally:
            sdc.kernel_timing(False)
        assert "grad_w_mfma" in ran, ran
        e = rel_l2(gw, ref)
        ec = max(rel_l2(gw[c], ref[c]) for c in range(wl.Co))
        _say(f"  xk {xdt}: gw {e:.3e} (worst channel {ec:.3e})")
        # bf16 X_K is exact in bf16: only the float32 accumulation order differs
        assert e <= (TOL if xdt == "bf16" else 2e-2) and ec <= (2e-5 if xdt == "bf16" else 3e-2)


@pytest.mark.parametrize("wl", CASES, ids=[c.name for c in CASES])
def test_fused_backward(sdc, wl):
    _say("fused backward", wl.name)
    x, w, gy = _inputs(wl)
    d = _desc(wl)
    gx_ref, gw_ref = oracle.backward(d, x, w, gy, wl.groups)
    psi = _psi(sdc, wl)
    gyd = torch.from_numpy(gy).cuda()
    sdc.kernel_timing(True)
    try:
        gx, gw, gb = sdc.fused_bwd(psi, _dev(x, wl.dtype), _dev(w, wl.dtype), gyd,
                                   groups=wl.groups, need_gbias=True)
        ran = set(sdc.kernel_timing_read())
    finally:
        sdc.kernel_timing(False)
    if wl.Ci // wl.groups == 1:
        # one input channel per group: grad_w straight from x and gy, no X_K
        assert "grad_w_depthwise" in ran and "contract_kernel" not in ran, ran
        # stride 1 or 2 with nlon_in = s nlon_out: grad_x on the register-tiled
        # folded kernel
        assert "contract_transpose_folded_tiled" in ran, ran
    e_x = rel_l2(gx.cpu().numpy(), gx_ref)
    e_w = rel_l2(gw.cpu().numpy(), gw_ref)
    e_b = rel_l2(gb.cpu().numpy(), gy.astype(np.float64).sum(axis=(0, 2, 3)))
    _say(f"  gx {e_x:.3e} gw {e_w:.3e} gbias {e_b:.3e}")
    assert e_x <= TOL and e_w <= TOL and e_b <= TOL
    # one gradient at a time gives the same values
    gx2, gw2, gb2 = sdc.fused_bwd(psi, _dev(x, wl.dtype), _dev(w, wl.dtype), gyd,
                                  groups=wl.groups, need_gw=False)
    assert gw2 is None and gb2 is None
    assert torch.equal(gx2, gx)
    _, gw3, _ = sdc.fused_bwd(psi, _dev(x, wl.dtype), _dev(w, wl.dtype), gyd, groups=wl.groups,
                              need_gx=False)
    assert torch.equal(gw3, gw)


# bf16 layers with spectral tables (stride 1, or 2 at 720 / 1440 longitudes)
# and a bf16 gradient: grad_x takes the longitude-spectral kernels (the
# adjoint of each window's circular correlation is a circular convolution:
# Psi_hat instead of its conjugate, the transposed window lists, the weights
# read transposed), held to the bf16 bar; grad_w runs on the matrix cores
# (split-K over points, X_K rounded to bf16 as it is loaded), also the bf16 bar
SPECTRAL_BWD = [
    W("spec_c4_like", 1, 64, 64, 1, 61, 120, 61, 120, (3, 3), 4 * math.pi / 60, "bf16"),
    W("spec_n720_co32_b2", 2, 128, 32, 1, 11, 720, 11, 720, (3,), 0.6, "bf16"),
    W("spec_lat_up", 1, 64, 96, 1, 21, 96, 41, 96, (3, 3), 0.5, "bf16"),
    # stride 2 (zeros inserted between gy's samples, then the stride-1
    # adjoint): 720 -> 360 and 1440 -> 720 longitudes
    W("spec_s2_720", 1, 64, 32, 1, 61, 720, 31, 360, (3, 3), 4 * math.pi / 30, "bf16"),
    W("spec_s2_1440", 1, 64, 32, 1, 25, 1440, 13, 720, (3,), 0.3, "bf16"),
]


@pytest.mark.parametrize("wl", SPECTRAL_BWD, ids=[c.name for c in SPECTRAL_BWD])
def test_fused_backward_spectral_grad_x(sdc, wl):
    _say("spectral grad_x", wl.name)
    x, w, gy = _inputs(wl)
    gy = round_bf16(gy)
    d = _desc(wl)
    gx_ref, gw_ref = oracle.backward(d, x, w, gy, wl.groups)
    psi = _psi(sdc, wl)
    gyd = _dev(gy, "bf16")
    sdc.kernel_timing(True)
    try:
        gx, gw, _ = sdc.fused_bwd(psi, _dev(x, "bf16"), _dev(w, "bf16"), gyd)
        ran = set(sdc.kernel_timing_read())
    finally:
        sdc.kernel_timing(False)
    assert "spec_mfma" in ran and "contract_transpose" not in ran, ran
    assert "grad_w_mfma" in ran and "grad_w_partial" not in ran, ran
    # X_K recomputed whole in bf16 on the matrix cores, not in float32 slabs
    assert "contract_mfma" in ran and "contract_kernel" not in ran, ran
    gx = gx.cpu().numpy()
    e_x = rel_l2(gx, gx_ref)
    gw = gw.cpu().numpy()
    e_w = rel_l2(gw, gw_ref)
    # per output channel of gw
    e_wc = max(rel_l2(gw[c], gw_ref[c]) for c in range(wl.Co))
    # per input row, so that an error confined to a few rows shows
    rows = [float(np.linalg.norm(gx[:, :, i] - gx_ref[:, :, i]) /
                  max(np.linalg.norm(gx_ref[:, :, i]), 1e-300)) for i in range(wl.nlat_in)]
    _say(f"  gx {e_x:.3e} (worst row {max(rows):.3e}) gw {e_w:.3e} (worst channel {e_wc:.3e})")
    assert e_x <= 2e-2 and max(rows) <= 3e-2
    # grad_w on the matrix cores: X_K rounded to bf16 (the bf16 bar)
    assert e_w <= 2e-2 and e_wc <= 3e-2
    # bf16 gx: the same sums, rounded once on store
    gx16, _, _ = sdc.fused_bwd(psi, _dev(x, "bf16"), _dev(w, "bf16"), gyd, need_gw=False,
                               gx_dtype=torch.bfloat16)
    assert gx16.dtype == torch.bfloat16
    assert rel_l2(gx16.float().cpu().numpy(), gx) <= 4e-3
    # a float32 gradient keeps the float32 path (exact to the float32 bar)
    gx32, _, _ = sdc.fused_bwd(psi, _dev(x, "bf16"), _dev(w, "bf16"), torch.from_numpy(gy).cuda(),
                               need_gw=False)
    assert rel_l2(gx32.cpu().numpy(), gx_ref) <= TOL


def test_fused_backward_slabs_and_full_ring_windows(sdc):
    # 181 x 360 at 64 channels, K = 7: the two slab tensors of the whole layer
    # take more than 64 MiB, so X_K is recomputed in 8 slabs of 23 rows; the
    # polar rows' windows span the whole ring
    wl = W("slabs", 1, 64, 32, 1, 181, 360, 181, 360, (3, 3), 4 * math.pi / 180, "bf16")
    assert 2 * wl.B * wl.Ci * wl.K * wl.nlon_out * 4 * wl.nlat_out > 64 << 20
    x, w, gy = _inputs(wl)
    d = _desc(wl)
    gx_ref, gw_ref = oracle.backward(d, x, w, gy, 1)
    psi = _psi(sdc, wl)
    gx, gw, _ = sdc.fused_bwd(psi, _dev(x, "bf16"), _dev(w, "bf16"), torch.from_numpy(gy).cuda())
    e_x, e_w = rel_l2(gx.cpu().numpy(), gx_ref), rel_l2(gw.cpu().numpy(), gw_ref)
    _say(f"slabs: gx {e_x:.3e} gw {e_w:.3e}")
    assert e_x <= TOL and e_w <= TOL


def test_unfused_backward_composes_to_fused(sdc):
    # the pages' fused=False backward: the saved X_K, then the adjoints
    wl = CASES[2]
    x, w, gy = _inputs(wl)
    psi = _psi(sdc, wl)
    xd, wd, gyd = _dev(x, "f32"), _dev(w, "f32"), torch.from_numpy(gy).cuda()
    xk = sdc.contract(psi, xd)
    gw_u = sdc.einsum_grad_w(xk, gyd, groups=wl.groups)
    gx_u = sdc.contract_transpose(psi, sdc.einsum_grad_xk(gyd, wd, groups=wl.groups))
    gx_f, gw_f, _ = sdc.fused_bwd(psi, xd, wd, gyd, groups=wl.groups)
    assert rel_l2(gx_u.cpu().numpy(), gx_f.cpu().numpy()) <= 1e-6
    assert rel_l2(gw_u.cpu().numpy(), gw_f.cpu().numpy()) <= 1e-6


def test_backward_empty_batch_and_errors(sdc):
    wl = CASES[0]
    psi = _psi(sdc, wl)
    x = torch.zeros((0, wl.Ci, wl.nlat_in, wl.nlon_in), device="cuda")
    w = torch.ones((wl.Co, wl.Ci, wl.K), device="cuda")
    gy = torch.zeros((0, wl.Co, wl.nlat_out, wl.nlon_out), device="cuda")
    gx, gw, gb = sdc.fused_bwd(psi, x, w, gy, need_gbias=True)
    assert gx.shape[0] == 0
    assert torch.count_nonzero(gw).item() == 0 and torch.count_nonzero(gb).item() == 0
    xk = torch.zeros((0, wl.Ci, wl.K, wl.nlat_out, wl.nlon_out), device="cuda")
    assert torch.count_nonzero(sdc.einsum_grad_w(xk, gy)).item() == 0
    with pytest.raises(ValueError):
        sdc.fused_bwd(psi, x, w, gy, need_gx=False, need_gw=False)
    with pytest.raises(ValueError):     # groups must divide the channels
        sdc.einsum_grad_w(torch.zeros((1, 3, wl.K, 2, 2), device="cuda"),
                          torch.zeros((1, 4, 2, 2), device="cuda"), groups=2)
    # gradient output aliasing an input
    xk1 = torch.zeros((1, wl.Ci, wl.K, wl.nlat_out, wl.nlon_out), device="cuda")
    with pytest.raises(ValueError):
        sdc.contract_transpose(psi, xk1, gx=xk1.view(-1)[:wl.Ci * wl.nlat_in * wl.nlon_in]
                               .view(1, wl.Ci, wl.nlat_in, wl.nlon_in))


def test_backward_deterministic(sdc):
    wl = CASES[7]
    x, w, gy = _inputs(wl)
    psi = _psi(sdc, wl)
    a = sdc.fused_bwd(psi, _dev(x, "bf16"), _dev(w, "bf16"), torch.from_numpy(gy).cuda())
    b = sdc.fused_bwd(psi, _dev(x, "bf16"), _dev(w, "bf16"), torch.from_numpy(gy).cuda())
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_full_size_c4_backward_channel_subsets(sdc):
    """721x1440, 128 -> 128 channels, K = 7, bf16 inputs: the fused backward
    on the whole layer; the oracle evaluates whole gradients on subsets of
    channels (gx of 3 input channels, gw of 3 x 3 channel pairs)."""
    wl = WORKLOADS["c4"]
    _say("full-size c4 backward")
    x, w, gy = _inputs(wl)
    d = _desc(wl)
    csr = oracle.psi(d)
    psi = _psi(sdc, wl)
    gx, gw, gb = sdc.fused_bwd(psi, _dev(x, "bf16"), _dev(w, "bf16"), torch.from_numpy(gy).cuda(),
                               need_gbias=True)
    torch.cuda.synchronize()
    ci_sub, co_sub = [0, 61, 127], [5, 64, 126]
    # gx[:, ci] = contract^T(sum_co w[co, ci, k] gy[co]) for the chosen ci
    gxk = oracle.einsum_grad_xk(gy, w[:, ci_sub, :], 1)
    gx_ref = oracle.contract_transpose(d, gxk, csr=csr)
    e_x = rel_l2(gx[:, ci_sub].cpu().numpy(), gx_ref)
    # gw[co, ci, k] = sum gy[co] X_K[ci, k]
    xk = oracle.contract(d, x[:, ci_sub], csr=csr)
    gw_ref = oracle.einsum_grad_w(gy[:, co_sub], xk, 1)
    e_w = rel_l2(gw[co_sub][:, ci_sub].cpu().numpy(), gw_ref)
    e_b = rel_l2(gb.cpu().numpy(), gy.astype(np.float64).sum(axis=(0, 2, 3)))
    _say(f"  c4 gx {e_x:.3e} gw {e_w:.3e} gbias {e_b:.3e}")
    assert e_x <= TOL and e_w <= TOL and e_b <= TOL


def test_full_size_c4_backward_bf16_gradient_grad_w(sdc):
    """721x1440, 128 -> 128 channels, K = 7, bf16 inputs and a bf16 gradient:
    the fused backward recomputes the whole X_K in bf16 on the matrix cores
    and sums grad_w there; the oracle evaluates gw on 3 x 3 channel pairs
    (the bf16 bar, whole and per output channel)."""
    wl = WORKLOADS["c4"]
    _say("full-size c4 backward, bf16 gradient: grad_w")
    x, w, gy = _inputs(wl)
    gy = round_bf16(gy)
    d = _desc(wl)
    psi = _psi(sdc, wl)
    sdc.kernel_timing(True)
    try:
        _, gw, _ = sdc.fused_bwd(psi, _dev(x, "bf16"), _dev(w, "bf16"), _dev(gy, "bf16"),
                                 need_gx=False)
        ran = set(sdc.kernel_timing_read())
    finally:
        sdc.kernel_timing(False)
    assert "contract_mfma" in ran and "grad_w_mfma" in ran, ran
    assert "contract_kernel" not in ran, ran
    ci_sub, co_sub = [0, 61, 127], [5, 64, 126]
    xk = oracle.contract(d, x[:, ci_sub])
    gw_ref = oracle.einsum_grad_w(gy[:, co_sub], xk, 1)
    got = gw[co_sub][:, ci_sub].cpu().numpy()
    e_w = rel_l2(got, gw_ref)
    e_wc = max(rel_l2(got[c], gw_ref[c]) for c in range(len(co_sub)))
    _say(f"  c4 gw {e_w:.3e} (worst channel {e_wc:.3e})")
    assert e_w <= 2e-2 and e_wc <= 3e-2


def test_full_size_c4_spectral_grad_x_channel_subsets(sdc):
    """721x1440, 128 -> 128 channels, K = 7, bf16 inputs and a bf16 gradient:
    grad_x on the longitude-spectral kernels for the whole layer; the oracle
    evaluates the adjoint on 3 input channels (bf16 bar, whole and per input
    row)."""
    wl = WORKLOADS["c4"]
    _say("full-size c4 spectral grad_x")
    x, w, gy = _inputs(wl)
    gy = round_bf16(gy)
    d = _desc(wl)
    csr = oracle.psi(d)
    psi = _psi(sdc, wl)
    sdc.kernel_timing(True)
    try:
        gx, _, _ = sdc.fused_bwd(psi, _dev(x, "bf16"), _dev(w, "bf16"), _dev(gy, "bf16"),
                                 need_gw=False)
        ran = set(sdc.kernel_timing_read())
    finally:
        sdc.kernel_timing(False)
    assert "spec_mfma" in ran and "contract_transpose" not in ran, ran
    ci_sub = [0, 61, 127]
    gxk = oracle.einsum_grad_xk(gy, w[:, ci_sub, :], 1)
    gx_ref = oracle.contract_transpose(d, gxk, csr=csr)
    got = gx[:, ci_sub].cpu().numpy()
    e_x = rel_l2(got, gx_ref)
    rows = [float(np.linalg.norm(got[:, :, i] - gx_ref[:, :, i]) /
                  max(np.linalg.norm(gx_ref[:, :, i]), 1e-300)) for i in range(wl.nlat_in)]
    _say(f"  c4 spectral gx {e_x:.3e} (worst row {max(rows):.3e})")
    assert e_x <= 2e-2 and max(rows) <= 3e-2


@pytest.mark.parametrize("wl", [CASES[0], CASES[1], CASES[6]],
                         ids=[CASES[0].name, CASES[1].name, CASES[6].name])
def test_fused_backward_spectral_grad_x_f32(sdc, wl):
    """float32 stride-1 layers with a float32 gradient: grad_x on the float32
    spectral kernels (float32 spectra), held to the float32 bar."""
    x, w, gy = _inputs(wl)
    d = _desc(wl)
    gx_ref, _ = oracle.backward(d, x, w, gy, wl.groups)
    psi = _psi(sdc, wl)
    sdc.kernel_timing(True)
    try:
        gx, _, _ = sdc.fused_bwd(psi, _dev(x, "f32"), _dev(w, "f32"), torch.from_numpy(gy).cuda(),
                                 need_gw=False)
        ran = set(sdc.kernel_timing_read())
    finally:
        sdc.kernel_timing(False)
    assert "spec32_conv" in ran and "contract_transpose" not in ran, ran
    e = rel_l2(gx.cpu().numpy(), gx_ref)
    _say(f"spectral float32 grad_x {wl.name}: {e:.3e}")
    assert e <= TOL
