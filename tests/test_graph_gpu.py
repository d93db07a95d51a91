"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay must equal the eager result bit for bit.

The fused call's spectral path allocates and frees its workspace with
stream-ordered allocation, which a graph records as allocation nodes; the
library issues no memset.  Replays are separated by eager work and
synchronisations, and the output is cleared with a fill kernel before each.
"""
import os

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


def _capture_and_replay(fn, out, replays=4):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(replays):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        _ = float(out.float().abs().sum().item())   # eager work between replays
    return ref


@pytest.mark.parametrize("path", ["spectral", "toeplitz"])
def test_fused_forward_in_a_graph(sdc, path, monkeypatch):
    if path == "toeplitz":
        monkeypatch.setenv("DISCO_FUSED_PATH", "toeplitz")
    else:
        monkeypatch.delenv("DISCO_FUSED_PATH", raising=False)
    # 96 longitudes: a multiple of 8, so the direct matrix-core kernel has its
    # tap tables, and 48 = 2^4 3 for the spectral transforms
    wl = Workload("graph", 21, 1, 64, 128, 1, 25, 96, 25, 96, (3, 3), oracle.num_basis((3, 3)),
                  0.45, "bf16")
    x, w = draw_inputs(wl)
    x, w = round_bf16(x), round_bf16(w)
    xd = torch.from_numpy(x).cuda().to(torch.bfloat16)
    wd = torch.from_numpy(w).cuda().to(torch.bfloat16)
    psi = sdc.psi_build(25, 96, 25, 96, (3, 3), 0.45).to_device()
    assert sdc.fused_is_spectral(psi, torch.bfloat16, 64, 128, 1) == (path == "spectral")
    y = torch.empty(1, 128, 25, 96, device="cuda")
    # the eager call runs the kernel the path names
    sdc.kernel_timing(True)
    try:
        sdc.fused_fwd(psi, xd, wd, y=y)
        names = set(sdc.kernel_timing_read())
    finally:
        sdc.kernel_timing(False)
    assert ("spec_mfma" if path == "spectral" else "fused_mfma") in names, names
    ref = _capture_and_replay(lambda: sdc.fused_fwd(psi, xd, wd, y=y), y)
    want = oracle.forward(oracle.Desc(25, 96, 25, 96, (3, 3), 0.45), x, w, 1)
    err = np.linalg.norm(ref.cpu().numpy() - want) / np.linalg.norm(want)
    assert err <= 2e-2


def test_contract_and_einsum_in_a_graph(sdc):
    # the bf16 contraction and the ring einsum (one group of 128 outputs)
    wl = Workload("graph2", 5, 1, 128, 128, 1, 33, 64, 33, 64, (3, 3), oracle.num_basis((3, 3)),
                  0.3, "bf16")
    x, w = draw_inputs(wl)
    x, w = round_bf16(x), round_bf16(w)
    xd = torch.from_numpy(x).cuda().to(torch.bfloat16)
    wd = torch.from_numpy(w).cuda().to(torch.bfloat16)
    psi = sdc.psi_build(33, 64, 33, 64, (3, 3), 0.3).to_device()
    xk = torch.empty(1, 128, wl.K, 33, 64, device="cuda", dtype=torch.bfloat16)
    y = torch.empty(1, 128, 33, 64, device="cuda")
    sdc.kernel_timing(True)
    try:
        sdc.contract(psi, xd, xk=xk)
        sdc.einsum(xk, wd, y=y)
        names = set(sdc.kernel_timing_read())
    finally:
        sdc.kernel_timing(False)
    assert {"contract_mfma", "einsum_ring_bf16"} <= names, names

    def both():
        sdc.contract(psi, xd, xk=xk)
        sdc.einsum(xk, wd, y=y)

    ref = _capture_and_replay(both, y)
    want = oracle.forward(oracle.Desc(33, 64, 33, 64, (3, 3), 0.3), x, w, 1)
    err = np.linalg.norm(ref.cpu().numpy() - want) / np.linalg.norm(want)
    assert err <= 2e-2
