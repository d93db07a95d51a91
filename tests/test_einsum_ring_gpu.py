"""GPU parity of the channel/basis contraction (the einsum of the forward
equation on the DiscreteContinuousConvS2 page) through the C ABI, for the
shapes its ring-pipelined kernel takes (one channel group of 64 or 128 output
channels, Ci K a multiple of 32, at least five or six 32-wide kappa steps,
nlat nlon a multiple of 8 and at least 256), against the float64 oracle.

X_K and the weights are bf16 values, so every product is exact in float32 and
only the float32 accumulation over Ci K terms rounds: float32 outputs are held
to relative L2 <= 1e-5, bf16 outputs to 8e-3 (one bf16 rounding).  The shapes
cover several output tiles per workgroup (more tiles than compute units), the
last tile of a batch shifted back over its neighbour, the smallest step count
the kernel accepts, batches above one, bias, and both output types.
"""
import sys

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


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


def _bf16_values(rng, shape, scale):
    a = torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * scale)
    return a.to(torch.bfloat16)


# (B, Ci, K, Co, H, W): H W = points per image
SHAPES = [
    (1, 128, 7, 128, 61, 120),     # a reduced 128-channel, 7-basis layer: 29 tiles
    (2, 32, 5, 128, 200, 150),     # 5 kappa steps, the least at 128 channels; 118 tiles
                                   # per image, the last one shifted
    (3, 64, 3, 64, 100, 96),       # 6 kappa steps, the least at 64 channels; 38 tiles each
    (1, 64, 3, 64, 16, 16),        # one tile exactly
    (2, 64, 7, 64, 181, 360),      # 255 tiles per image: 510 tiles over the compute units
]


def _case(shape, seed):
    B, Ci, K, Co, H, W = shape
    rng = np.random.default_rng(seed)
    xk = _bf16_values(rng, (B, Ci, K, H, W), 1.0)
    w = _bf16_values(rng, (Co, Ci, K), 1.0 / np.sqrt(Ci * K))
    bias = torch.from_numpy(np.linspace(-1, 1, Co).astype(np.float32))
    return xk, w, bias


@pytest.mark.parametrize("shape", SHAPES, ids=["x".join(map(str, s)) for s in SHAPES])
def test_einsum_ring(sdc, shape, monkeypatch):
    monkeypatch.delenv("DISCO_EINSUM_PATH", raising=False)
    _say("einsum ring", shape)
    xk, w, bias = _case(shape, sum(shape))
    ref = oracle.einsum(xk.float().numpy(), w.float().numpy(), 1)
    refb = ref + bias.numpy().astype(np.float64)[None, :, None, None]
    xd, wd, bd = xk.cuda(), w.cuda(), bias.cuda()
    sdc.kernel_timing(True)
    try:
        y = sdc.einsum(xd, wd).cpu().numpy()
        names = sdc.kernel_timing_read()
    finally:
        sdc.kernel_timing(False)
    assert list(names) == ["einsum_ring_bf16"]
    err = rel_l2(y, ref)
    _say(f"  f32 rel-L2 {err:.3e}")
    assert err <= 1e-5
    yb = sdc.einsum(xd, wd, bias=bd).cpu().numpy()
    assert rel_l2(yb, refb) <= 1e-5
    yh = sdc.einsum(xd, wd, bias=bd, out_dtype=torch.bfloat16).float().cpu().numpy()
    errh = rel_l2(yh, refb)
    _say(f"  bf16-out rel-L2 {errh:.3e}")
    assert errh <= 8e-3
    # the double-buffered kernel against the oracle on the same inputs
    monkeypatch.setenv("DISCO_EINSUM_PATH", "stream")
    sdc.kernel_timing(True)
    try:
        ys = sdc.einsum(xd, wd, bias=bd).cpu().numpy()
        names = sdc.kernel_timing_read()
    finally:
        sdc.kernel_timing(False)
    assert list(names) == ["einsum_stream_bf16"]
    assert rel_l2(ys, refb) <= 1e-5


def test_einsum_ring_deterministic(sdc, monkeypatch):
    # the shifted last tile rewrites its neighbour's columns with the same values
    monkeypatch.delenv("DISCO_EINSUM_PATH", raising=False)
    xk, w, _ = _case(SHAPES[1], 5)
    xd, wd = xk.cuda(), w.cuda()
    a = sdc.einsum(xd, wd).cpu().numpy()
    b = sdc.einsum(xd, wd).cpu().numpy()
    assert np.array_equal(a, b)


def test_einsum_small_grids_take_other_kernels(sdc, monkeypatch):
    # fewer than 256 points, or too few kappa steps: the double-buffered kernel
    monkeypatch.delenv("DISCO_EINSUM_PATH", raising=False)
    for shape in [(1, 64, 7, 64, 8, 24), (1, 32, 3, 64, 32, 64)]:
        xk, w, _ = _case(shape, 3)
        ref = oracle.einsum(xk.float().numpy(), w.float().numpy(), 1)
        sdc.kernel_timing(True)
        try:
            y = sdc.einsum(xk.cuda(), w.cuda()).cpu().numpy()
            names = sdc.kernel_timing_read()
        finally:
            sdc.kernel_timing(False)
        assert "einsum_ring_bf16" not in names
        assert rel_l2(y, ref) <= 1e-5
