"""Benchmark of the forward DISCO convolution on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4] [--no-cpu-baseline]
    python bench.py --copy-calibration      (one plain device copy of known size, for
                                             calibrating rocprofv3 FETCH_SIZE / WRITE_SIZE)

A step is one forward pass (one disco_fused_fwd call: contraction and
channel/basis contraction without storing the K-expanded tensor) over one
batch of seeded synthetic input that is resident in device memory before
timing starts.  Psi is built once before
the timed region (it is a precomputed tensor of the layer).  The unfused pair
(contraction writing the K-expanded tensor, then the channel/basis GEMM) is
timed alongside and reported as extra fields.

Prints one JSON line.  `value` is output points x output channels per second.
`roofline` prices the fused kernel's algorithmic work (channel/basis FLOPs
plus 2 FLOPs per non-zero Psi entry, channel and output longitude) against
the MI355X dense bf16 matrix peak (2.5 PFLOP/s) or, for float32 workloads,
the float32 peak (157.3 TFLOP/s).  `cpu_baseline` is the float64 CPU oracle
timed on a bounded sample of output rows of the same workload, single-threaded,
and extrapolated to the whole workload by support-point weighting (the oracle's
time is linear in the support size of the rows it evaluates).

The timed unit of the fused forward is one disco_fused_fwd call.  For layers
the longitude-spectral algorithm takes (the headline workload is one) a call is
four launches: weight tiling, the forward real DFT of x, the per-frequency
window and channel/basis matrix-core kernel (spec_mfma), and the inverse real
DFT; for others it is the weight tiling and the direct fused kernel.

`roofline` describes the call's dominant kernel.  A second pass over the same
inputs records HIP events around every launch on its stream (the library's
disco_kernel_timing); the kernel with the largest total is priced against its
own algorithmic work per launch (spec_mfma: its product and window-sum flops;
the direct kernel: the method's flops).  `kernels_ms` lists every kernel's
average, and `call_roofline` prices the whole call on the method's algorithmic
flops.  The direct kernel's time on the same inputs is `direct_fused_ms`.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
HBM_PEAK_GBS = 8000.0

METRIC = "DISCO fwd output-points\u00b7Cout/s at 721x1440 C=128 K=7; % HBM/MFMA roofline"

# rocprofv3 HBM counters at the headline workload, per launch of a kernel or
# per call (summed over the call's launches): FETCH_SIZE x 2.000 + WRITE_SIZE
# x 1.000 (factors from a 512 MiB device copy, see profiles/).  Keyed by the SHA-1 of the kernel source
# the counters were taken with: when the source has changed the figure is
# stale and `traffic` is reported as null.
MEASURED_TRAFFIC_BYTES = {
    ("c4", "fused_spectral"): {"bytes": 2041565112, "source": "kernels_spectral.hip",
                               "sha1": "0b83d543098c288513e3306217d414739f9e5c56"},
    ("c4", "spec_mfma"): {"bytes": 699515569, "source": "kernels_spectral.hip",
                          "sha1": "0b83d543098c288513e3306217d414739f9e5c56"},
    ("c4", "fused"): {"bytes": 1377027391, "source": "kernels_fused_mfma.hip",
                      "sha1": "d3a7660ad665af7d9a8ccdb85b7aff879512fa4e"},
    ("c4", "contract"): {"bytes": 2870807783, "source": "kernels_fused_mfma.hip",
                         "sha1": "d3a7660ad665af7d9a8ccdb85b7aff879512fa4e"},
    ("c4", "einsum"): {"bytes": 2437461650, "source": "kernels_einsum_mfma.hip",
                       "sha1": "4683e91365bc9e8ddd3298a6ec541ce2c779c88c"},
}
CSRC = os.path.join(ROOT, "spherical_disco_convolution_amd", "csrc")


def measured_traffic(key, kernel, grid="equiangular"):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE (copy-calibrated),
    or None when there is no figure or the kernel source changed since it was taken."""
    import hashlib
    m = MEASURED_TRAFFIC_BYTES.get((key, kernel)) if grid == "equiangular" else None
    src = os.path.join(CSRC, m["source"]) if m else None
    if m is None or not os.path.exists(src):
        return None
    with open(src, "rb") as f:
        sha = hashlib.sha1(f.read()).hexdigest()
    return m["bytes"] if sha == m["sha1"] else None

COPY_CALIBRATION_BYTES = 512 << 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="c1..c5 (default: the headline case c4)")
    ap.add_argument("--grid", default="equiangular",
                    choices=["equiangular", "legendre-gauss", "lobatto", "equiangular-trapezoidal"],
                    help="latitude grid of input and output (default: equiangular, the "
                         "workloads' own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unfused", action="store_true")
    ap.add_argument("--fused-only", action="store_true", help="time only the fused kernel (profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one device-to-device copy of %d MiB and exit" % (COPY_CALIBRATION_BYTES >> 20))
    return ap.parse_args()


def copy_calibration():
    """One plain copy of known size: FETCH_SIZE and WRITE_SIZE of its kernel
    divided into COPY_CALIBRATION_BYTES give the counters' scale factors."""
    import torch
    n = COPY_CALIBRATION_BYTES // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_CALIBRATION_BYTES,
                      "read_bytes": COPY_CALIBRATION_BYTES, "write_bytes": COPY_CALIBRATION_BYTES}),
          flush=True)


def algorithmic_flops(wl, nnz_nonzero):
    """Channel/basis FLOPs + 2 per non-zero Psi entry per channel and output longitude."""
    f_einsum = 2.0 * wl.B * wl.Co * (wl.Ci // wl.groups) * wl.K * wl.nlat_out * wl.nlon_out
    f_contr = 2.0 * wl.B * wl.Ci * wl.nlon_out * nnz_nonzero
    return f_einsum, f_contr


def spec_mfma_flops(wl, windows):
    """Algorithmic flops of one spec_mfma launch: the channel/basis product over
    the real and imaginary parts of frequencies 0..N/2 (2 Co Ci K per output
    row entry), plus one complex multiply-add (8 flops) per channel, window,
    basis function and frequency of the window sum."""
    M = wl.nlon_out // 2 + 1
    gemm = 2.0 * wl.B * wl.Co * wl.Ci * wl.K * wl.nlat_out * 2 * M
    window = 8.0 * wl.B * wl.Ci * windows * wl.K * M
    return gemm + window


def count_windows(psi):
    """(output row, input row) pairs of Psi's support: the windows."""
    import numpy as np
    row_ptr, in_lat, _, _ = psi.export()
    rows = np.repeat(np.arange(len(row_ptr) - 1), np.diff(row_ptr))
    return int(len(np.unique(rows.astype(np.int64) * (1 << 20) + in_lat)))


def algorithmic_bytes(wl, nnz_support, dsize):
    x = wl.B * wl.Ci * wl.nlat_in * wl.nlon_in * dsize
    w = wl.Co * (wl.Ci // wl.groups) * wl.K * dsize
    psi = nnz_support * (8 + 4 * wl.K)
    y = wl.B * wl.Co * wl.nlat_out * wl.nlon_out * 4
    return x + w + psi + y


def time_region(fn, steps, torch):
    """Wall time and HIP-event time of `steps` calls of fn on the current stream."""
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) / 1000.0


def cpu_baseline(wl, x, w, grid="equiangular"):
    import oracle
    from threadpoolctl import threadpool_limits
    d = oracle.Desc(wl.nlat_in, wl.nlon_in, wl.nlat_out, wl.nlon_out, wl.kernel_shape,
                    wl.theta_cutoff, grid_in=grid, grid_out=grid)
    csr = oracle.psi(d)
    # systematic sample of output rows, all longitudes, batches and channels:
    # up to 60 rows, fewer where the oracle's estimated time would pass about
    # 30 s (its time per support point grows with B * Ci * K * nlon_out; about
    # 6e8 of those units per second on one core, from the 721x1440 sample)
    units = wl.B * wl.Ci * wl.K * wl.nlon_out * csr.nnz / wl.nlat_out
    n_rows = int(max(2, min(60, 30.0 * 6e8 / max(units, 1.0))))
    step = max(1, wl.nlat_out // n_rows)
    rows = list(range(step // 2, wl.nlat_out, step))
    sup = sum(int(csr.row_ptr[j + 1] - csr.row_ptr[j]) for j in rows)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.forward(d, x, w, wl.groups, csr=csr, rows=rows)
        dt = time.perf_counter() - t0
    pts = wl.B * len(rows) * wl.nlon_out * wl.Co
    # the oracle's time is linear in the support it evaluates: extrapolate the
    # sample to the whole workload by support weighting
    t_all = dt * csr.nnz / sup
    total_pts = wl.B * wl.nlat_out * wl.nlon_out * wl.Co
    return {
        "value": total_pts / t_all,
        "unit": "output-points\u00b7Cout/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{len(rows)} of {wl.nlat_out} output rows (every {step}th from {step // 2}), "
                   f"all longitudes, batches and channels, {sup} of {csr.nnz} support points; "
                   f"float64 numpy, BLAS limited to 1 thread; {dt:.1f} s, i.e. {pts / dt:.3g} "
                   f"output-points\u00b7Cout/s on the sample, extrapolated by support to "
                   f"{t_all:.0f} s for the whole workload"),
    }


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 "
                          "(multi-GPU sharding is described, not implemented)"}), flush=True)
        sys.exit(2)
    import numpy as np
    import torch

    import spherical_disco_convolution_amd as sdc
    from disco_workloads import HEADLINE, WORKLOADS, draw_inputs, round_bf16

    key = args.workload or HEADLINE
    wl = WORKLOADS[key]
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    torch.cuda.set_device(0)

    x, w = draw_inputs(wl)
    if wl.dtype == "bf16":
        x, w = round_bf16(x), round_bf16(w)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    xd = torch.from_numpy(x).cuda().to(tdt).contiguous()
    wd = torch.from_numpy(w).cuda().to(tdt).contiguous()

    t0 = time.perf_counter()
    psi = sdc.psi_build(wl.nlat_in, wl.nlon_in, wl.nlat_out, wl.nlon_out, wl.kernel_shape,
                        wl.theta_cutoff, grid_in=args.grid, grid_out=args.grid)
    psi_build_s = time.perf_counter() - t0
    t0 = time.perf_counter()
    psi.to_device()
    torch.cuda.synchronize()
    psi_upload_s = time.perf_counter() - t0
    spectral = sdc.fused_is_spectral(psi, tdt, wl.Ci, wl.Co, wl.groups)

    y = torch.empty((wl.B, wl.Co, wl.nlat_out, wl.nlon_out), dtype=torch.float32, device="cuda")
    fused = lambda: sdc.fused_fwd(psi, xd, wd, groups=wl.groups, y=y)

    for _ in range(args.warmup):
        fused()
    torch.cuda.synchronize()
    wall, ev = time_region(fused, args.steps, torch)
    ms_per_step = wall / args.steps * 1000.0
    kernel_s = ev / args.steps
    work = wl.out_points_cout
    value = work / (ms_per_step / 1000.0)

    f_einsum, f_contr = algorithmic_flops(wl, psi.nnz_nonzero)
    f_alg = f_einsum + f_contr
    cig = wl.Ci // wl.groups
    if cig == 1:
        # one input channel per group: weights fold into the taps per channel
        f_folded = 2.0 * wl.B * wl.Co * wl.nlon_out * psi.nnz + 2.0 * wl.Co * psi.nnz_nonzero
        f_alg = min(f_alg, f_folded)
    dsize = 2 if wl.dtype == "bf16" else 4
    peak = PEAK_TFLOPS[wl.dtype]
    achieved = f_alg / kernel_s / 1e12
    traffic = measured_traffic(key, "fused_spectral" if spectral else "fused", args.grid)
    call_roofline = {"bound": "mfma" if wl.dtype == "bf16" else "alu",
                     "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic}

    # per-kernel HIP events (a separate pass: the event records stay out of
    # the timed region above)
    sdc.kernel_timing(True)
    try:
        for _ in range(args.steps):
            fused()
        kt = sdc.kernel_timing_read()
    finally:
        sdc.kernel_timing(False)
    kernels_ms = {k: round(tot / n, 4) for k, (tot, n) in kt.items()}
    dom = max(kt, key=lambda k: kt[k][0])
    dom_s = kt[dom][0] / kt[dom][1] / 1000.0
    if dom == "spec_mfma":
        f_dom = spec_mfma_flops(wl, count_windows(psi))
    else:
        f_dom = f_alg
    a_dom = f_dom / dom_s / 1e12
    roofline = {"bound": "mfma" if wl.dtype == "bf16" else "alu", "achieved": round(a_dom, 3),
                "peak": peak, "unit": "TFLOP/s", "frac": round(a_dom / peak, 4),
                "traffic": measured_traffic(key, dom, args.grid), "kernel": dom,
                "kernel_ms": round(dom_s * 1000, 4), "algorithmic_flop": f_dom}
    extra = {
        "fused_kernel_ms": round(kernel_s * 1000, 4),
        "kernels_ms": kernels_ms,
        "call_roofline": call_roofline,
        "algorithmic_flop": f_alg,
        "algorithmic_bytes": algorithmic_bytes(wl, psi.nnz, dsize),
        "hbm_GBps_algorithmic": round(algorithmic_bytes(wl, psi.nnz, dsize) / kernel_s / 1e9, 1),
        "psi_build_s": round(psi_build_s, 3),
        "psi_upload_s": round(psi_upload_s, 3),
    }
    extra["fused_algorithm"] = "spectral" if spectral else "direct"
    if not args.fused_only and spectral:
        # the direct matrix-core kernel on the same inputs, for comparison
        os.environ["DISCO_FUSED_PATH"] = "toeplitz"
        try:
            for _ in range(2):
                fused()
            _, t_s = time_region(fused, args.steps, torch)
            extra["direct_fused_ms"] = round(t_s / args.steps * 1000, 4)
        finally:
            del os.environ["DISCO_FUSED_PATH"]
    if not args.no_unfused and not args.fused_only:
        xk = torch.empty((wl.B, wl.Ci, wl.K, wl.nlat_out, wl.nlon_out), dtype=tdt, device="cuda")
        contract = lambda: sdc.contract(psi, xd, xk=xk)
        einsum = lambda: sdc.einsum(xk, wd, groups=wl.groups, y=y)
        for _ in range(2):
            contract()
            einsum()
        n = max(3, args.steps // 2)
        _, t_c = time_region(contract, n, torch)
        _, t_e = time_region(einsum, n, torch)
        extra["contract_ms"] = round(t_c / n * 1000, 4)
        extra["einsum_ms"] = round(t_e / n * 1000, 4)
        extra["unfused_ms"] = round((t_c + t_e) / n * 1000, 4)
        # both are HBM-bound: algorithmic bytes per launch over the launch time
        xk_bytes = wl.B * wl.Ci * wl.K * wl.nlat_out * wl.nlon_out * dsize
        a_bytes = algorithmic_bytes(wl, psi.nnz, dsize)
        x_psi = a_bytes - (wl.Co * cig * wl.K * dsize) - wl.B * wl.Co * wl.nlat_out * wl.nlon_out * 4
        b_contract = x_psi + xk_bytes
        b_einsum = xk_bytes + (a_bytes - x_psi)
        for name, nb, t in (("contract", b_contract, t_c / n), ("einsum", b_einsum, t_e / n)):
            gbps = nb / t / 1e9
            extra[name + "_roofline"] = {"bound": "hbm", "achieved": round(gbps, 1),
                                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                         "frac": round(gbps / HBM_PEAK_GBS, 4),
                                         "traffic": measured_traffic(key, name, args.grid)}
        del xk
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "output-points\u00b7Cout/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) input, N(0,1/(Ci*K)) weights)",
        "config": {"workload": f"{key}: B={wl.B} Ci={wl.Ci} Co={wl.Co} groups={wl.groups} "
                               f"{wl.nlat_in}x{wl.nlon_in}->{wl.nlat_out}x{wl.nlon_out} "
                               f"kernel_shape={wl.kernel_shape} K={wl.K} "
                               f"theta_cutoff={wl.theta_cutoff:.6f} {wl.dtype}, fused forward"
                               + ("" if args.grid == "equiangular" else f", {args.grid} grid"),
                   "global_batch": wl.B, "parallelism": "single GPU"},
        "roofline": roofline,
    }
    line.update(extra)
    if not args.no_cpu_baseline and not args.fused_only:
        line["cpu_baseline"] = cpu_baseline(wl, x, w, args.grid)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
