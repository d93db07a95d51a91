"""Benchmark of the forward DISCO convolution on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4] [--no-cpu-baseline]
    python bench.py --copy-calibration      (one plain device copy of known size, for
                                             calibrating rocprofv3 FETCH_SIZE / WRITE_SIZE)
    python bench.py --peaks                 (only the peak micro-benchmarks)

A step is one forward pass (one disco_fused_fwd call: contraction and
channel/basis contraction without storing the K-expanded tensor) over one
batch of seeded synthetic input that is resident in device memory before
timing starts.  Psi is built once before the timed region (it is a
precomputed tensor of the layer).  The unfused pair (contraction writing the
K-expanded tensor, then the channel/basis GEMM) is timed alongside and
reported as extra fields.

Prints one JSON line.  `value` is output points x output channels per second.

`roofline` prices the whole fused call: the method's algorithmic work per call
(channel/basis FLOPs plus 2 FLOPs per non-zero Psi entry, channel and output
longitude; for one input channel per group the smaller folded count) over the
call's time from HIP events on its launch stream (the timed region), against
the MI355X dense bf16 matrix peak (2.5 PFLOP/s) or, for float32 workloads, the
float32 peak (157.3 TFLOP/s).  A call is several launches (weight tiling,
transforms, the main kernels); `kernels_ms` gives each one's average from a
second pass with per-launch HIP events, and `dominant_kernel` prices the
largest of them on its own algorithmic work.  `traffic` is the call's HBM
bytes from rocprofv3 FETCH_SIZE and WRITE_SIZE (copy-calibrated), taken from
the profiles file named in `traffic_source` at the kernel source's SHA-1, or
null when the source has changed since.

`cpu_baseline` is the float64 CPU oracle on all the host cores this process
may use (at most 16, the GPU's share of the host), one worker process per
core, each evaluating whole output rows.  It runs the whole workload when
that is estimated to take at most about 30 s, otherwise a systematic sample
of output rows, extrapolated by support size (the oracle's time is linear in
the support it evaluates).  It runs before the GPU is touched.

`measured_peaks` are the machine's own HBM copy and read bandwidth, dense bf16
matrix-core rate and LDS read rate from hand-written micro-benchmarks
(libdisco_probe.so), beside the published peaks the roofline divides by.
`cold_ms` is the fused call after a 1 GiB write has flushed the caches.
`bwd_ms` / `bwd_grad_x_ms` time disco_fused_bwd (gradient in the layer's
dtype) for gx and gw, and for gx alone.

Warm-up: after idling, the GPU runs the first 30-40 back-to-back calls at
lower clocks (at 721x1440, 128 channels: 0.78-0.95 ms per call, settling to
0.68-0.70 ms); the default 50 untimed calls put the timed region in the
sustained state a serving or training loop runs in.
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

# rocprofv3 HBM counters per launch of a kernel or per call (summed over the
# call's launches): FETCH_SIZE x 2.000 + WRITE_SIZE x 1.000 (factors from a
# 512 MiB device copy, see profiles/).  Keyed by the SHA-1 of the kernel source
# the counters were taken with: when the source has changed the figure is
# stale and `traffic` is reported as null.
MEASURED_TRAFFIC_BYTES = {
    ("c4", "fused_spectral"): {"bytes": 2036857276, "source": "kernels_spectral.hip",
                  "sha1": "f89593bda0baf3412d31fb230ecd10cda17f66d6",
                  "profile": "profiles/c4_counters.md"},
    ("c4", "spec_mfma"): {"bytes": 694550282, "source": "kernels_spectral.hip",
                  "sha1": "f89593bda0baf3412d31fb230ecd10cda17f66d6",
                  "profile": "profiles/c4_counters.md"},
    ("c4", "fused"): {"bytes": 1373252505, "source": "kernels_fused_mfma.hip",
                  "sha1": "d0e9c723b5d451ca9066de577ecb6dd831f5ac82",
                  "profile": "profiles/c4_counters.md"},
    ("c4", "contract"): {"bytes": 2870729062, "source": "kernels_fused_mfma.hip",
                  "sha1": "d0e9c723b5d451ca9066de577ecb6dd831f5ac82",
                  "profile": "profiles/c4_counters.md"},
    ("c4", "einsum"): {"bytes": 2437672883, "source": "kernels_einsum_mfma.hip",
                  "sha1": "4683e91365bc9e8ddd3298a6ec541ce2c779c88c",
                  "profile": "profiles/c4_counters.md"},
    ("c3", "fused_spectral"): {"bytes": 381483442, "source": "kernels_spectral.hip",
                  "sha1": "f89593bda0baf3412d31fb230ecd10cda17f66d6",
                  "profile": "profiles/c3_counters.md"},
    ("c3", "spec_mfma"): {"bytes": 173069994, "source": "kernels_spectral.hip",
                  "sha1": "f89593bda0baf3412d31fb230ecd10cda17f66d6",
                  "profile": "profiles/c3_counters.md"},
    ("c5", "fused"): {"bytes": 1815006080, "source": "kernels_generic.hip",
                  "sha1": "19bd4e142e694c83a53b5b50c884c4000d29bdd2",
                  "profile": "profiles/c5_counters.md"},
    ("c5", "fused_depthwise"): {"bytes": 1815006080, "source": "kernels_generic.hip",
                  "sha1": "19bd4e142e694c83a53b5b50c884c4000d29bdd2",
                  "profile": "profiles/c5_counters.md"},
    ("c2", "fused_spectral"): {"bytes": 274472948, "source": "kernels_spectral.hip",
                  "sha1": "f89593bda0baf3412d31fb230ecd10cda17f66d6",
                  "profile": "profiles/c2_counters.md"},
    ("c2", "spec32_conv"): {"bytes": 200221482, "source": "kernels_spectral.hip",
                  "sha1": "f89593bda0baf3412d31fb230ecd10cda17f66d6",
                  "profile": "profiles/c2_counters.md"},
}
CSRC = os.path.join(ROOT, "spherical_disco_convolution_amd", "csrc")


def measured_traffic(key, kernel, grid="equiangular", with_source=False):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE (copy-calibrated),
    or None when there is no figure or the kernel source changed since it was taken.
    with_source: also return where the figure comes from (profiles file and the
    kernel source's SHA-1), or why it is null."""
    import hashlib
    m = MEASURED_TRAFFIC_BYTES.get((key, kernel)) if grid == "equiangular" else None
    src = os.path.join(CSRC, m["source"]) if m else None
    if m is None or not os.path.exists(src):
        out, why = None, "no counter figure for this workload and kernel"
    else:
        with open(src, "rb") as f:
            sha = hashlib.sha1(f.read()).hexdigest()
        if sha == m["sha1"]:
            out, why = m["bytes"], f"{m['profile']} ({m['source']} sha1 {m['sha1'][:12]})"
        else:
            out, why = None, (f"{m['profile']} was taken at {m['source']} sha1 {m['sha1'][:12]}; "
                              f"the source is now {sha[:12]}")
    return (out, why) if with_source else out

COPY_CALIBRATION_BYTES = 512 << 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU reaches its sustained clocks after about 30 back-to-back calls
    # (~25 ms of load); 50 untimed calls put the timed ones past that ramp
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None, help="c1..c5 (default: the headline case c4)")
    ap.add_argument("--grid", default="equiangular",
                    choices=["equiangular", "legendre-gauss", "lobatto", "equiangular-trapezoidal"],
                    help="latitude grid of input and output (default: equiangular, the "
                         "workloads' own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unfused", action="store_true")
    ap.add_argument("--no-bwd", action="store_true", help="skip the fused backward timing")
    ap.add_argument("--fused-only", action="store_true", help="time only the fused kernel (profiling)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the peak micro-benchmarks")
    ap.add_argument("--peaks", action="store_true",
                    help="run only the peak micro-benchmarks (HBM, matrix cores, LDS) and exit")
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
    """Algorithmic flops of one launch of the spectral product kernel
    (spec_mfma, or spec32_conv for float32): the channel/basis product over the
    real and imaginary parts of the input grid's frequencies 0..N_in/2 (2 Co Ci
    K per output row entry; a stride-2 layer folds them onto the output grid
    afterwards), plus one complex multiply-add (8 flops) per channel, window,
    basis function and frequency of the window sum."""
    M = wl.nlon_in // 2 + 1
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


# Arguments of the CPU-baseline workers, set in the parent before the pool
# forks (the children read them, copy-on-write; nothing is pickled).
_ORACLE_JOB = {}


def _oracle_rows(rows):
    """One worker's share of the CPU baseline: the oracle's forward pass over
    whole output rows, single-threaded."""
    import oracle
    from threadpoolctl import threadpool_limits
    j = _ORACLE_JOB
    with threadpool_limits(limits=1):
        oracle.forward(j["desc"], j["x"], j["w"], j["groups"], csr=j["csr"], rows=rows)
    return len(rows)


def host_cores():
    """Host cores this process may use, capped at 16 (the GPU's share of the
    host on a one-GPU machine)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(wl, x, w, grid="equiangular"):
    """The float64 oracle on this host's cores: one forked worker process per
    core, each evaluating whole output rows (largest first).  Must run before
    the GPU is initialised in this process (the workers are forked)."""
    import multiprocessing as mp
    import numpy as np
    import oracle
    d = oracle.Desc(wl.nlat_in, wl.nlon_in, wl.nlat_out, wl.nlon_out, wl.kernel_shape,
                    wl.theta_cutoff, grid_in=grid, grid_out=grid)
    t0 = time.perf_counter()
    csr = oracle.psi(d)
    psi_s = time.perf_counter() - t0
    cores = host_cores()
    sup = np.diff(csr.row_ptr).astype(np.float64)
    x64, w64 = np.asarray(x, np.float64), np.asarray(w, np.float64)
    # the oracle's time per support point grows with B * Ci * K * nlon_out:
    # its rate in those units on this host comes from one light row timed
    # here (single-threaded); the whole workload runs when that predicts at
    # most ~30 s on these cores, otherwise a systematic sample of rows
    from threadpoolctl import threadpool_limits
    probe = int(np.argmin(np.where(sup > 0, sup, np.inf)))
    per_point = wl.B * wl.Ci * wl.K * wl.nlon_out
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.forward(d, x64, w64, wl.groups, csr=csr, rows=[probe])
        rate = per_point * sup[probe] / max(time.perf_counter() - t0, 1e-6)
    est = per_point * float(sup.sum()) / rate / cores
    if est <= 30.0:
        rows = list(range(wl.nlat_out))
    else:
        n_rows = int(max(min(cores, wl.nlat_out), min(wl.nlat_out, wl.nlat_out * 30.0 / est)))
        step = max(1, wl.nlat_out // n_rows)
        rows = list(range(step // 2, wl.nlat_out, step))
    sample_sup = float(sup[rows].sum())
    # one task per row, heaviest first, so that the workers finish together
    tasks = [[r] for r in sorted(rows, key=lambda r: -sup[r])]
    # float64 once in the parent: the oracle's own conversion is then a no-op
    # in every task
    _ORACLE_JOB.update(desc=d, x=x64, w=w64, groups=wl.groups, csr=csr)
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        done = sum(pool.imap_unordered(_oracle_rows, tasks, chunksize=1))
    dt = time.perf_counter() - t0
    _ORACLE_JOB.clear()
    assert done == len(rows)
    whole = len(rows) == wl.nlat_out
    t_all = dt if whole else dt * float(sup.sum()) / sample_sup
    total_pts = wl.B * wl.nlat_out * wl.nlon_out * wl.Co
    if whole:
        sample = (f"the whole workload ({wl.nlat_out} output rows, all longitudes, batches and "
                  f"channels) in {dt:.1f} s")
    else:
        sample = (f"{len(rows)} of {wl.nlat_out} output rows (every {rows[1] - rows[0] if len(rows) > 1 else 1}th), "
                  f"all longitudes, batches and channels, {int(sample_sup)} of {int(sup.sum())} "
                  f"support points, in {dt:.1f} s; extrapolated by support to {t_all:.0f} s for "
                  f"the whole workload")
    return {
        "value": total_pts / t_all,
        "unit": "output-points\u00b7Cout/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"float64 numpy oracle, {cores} single-threaded worker processes (one per host "
                   f"core), one output row per task; " + sample +
                   f"; sample size from a timed single-core row ({rate:.3g} "
                   f"B*Ci*K*nlon_out units per support point per second)" +
                   f"; its Psi build took {psi_s:.1f} s (not included)"),
    }


def measure_peaks():
    """The machine's own rates from libdisco_probe.so: HBM copy and read
    bandwidth over 1 GiB buffers, dense bf16 matrix-core rate and LDS read
    rate (each the best of three launches' averages)."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "spherical_disco_convolution_amd", "libdisco_probe.so"))
    P, F, D, I = ctypes.c_void_p, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double), ctypes.c_int
    lib.probe_hbm_copy.argtypes = [P, P, ctypes.c_size_t, I, F]
    lib.probe_hbm_read.argtypes = [P, ctypes.c_size_t, P, I, F]
    lib.probe_mfma_bf16.argtypes = [P, I, I, I, F, D]
    lib.probe_lds_read.argtypes = [P, I, I, I, F, D]
    nbytes = 1 << 30
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    scratch = torch.zeros(1 << 20, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    ms = ctypes.c_float()
    amount = ctypes.c_double()

    def best(fn):
        t = []
        for _ in range(3):
            rc = fn()
            if rc != 0:
                raise RuntimeError(f"probe failed ({rc})")
            t.append(ms.value)
        return min(t)

    t_copy = best(lambda: lib.probe_hbm_copy(b.data_ptr(), a.data_ptr(), nbytes, 5, ctypes.byref(ms)))
    t_read = best(lambda: lib.probe_hbm_read(a.data_ptr(), nbytes, scratch.data_ptr(), 5,
                                             ctypes.byref(ms)))
    t_mfma = best(lambda: lib.probe_mfma_bf16(scratch.data_ptr(), 2, 4096, 3, ctypes.byref(ms),
                                              ctypes.byref(amount)))
    f_mfma = amount.value
    t_lds = best(lambda: lib.probe_lds_read(scratch.data_ptr(), 2, 2048, 3, ctypes.byref(ms),
                                            ctypes.byref(amount)))
    b_lds = amount.value
    ncu = lib.probe_num_cus()
    del a, b, scratch
    torch.cuda.empty_cache()
    lds_tbs = b_lds / (t_lds / 1e3) / 1e12
    return {
        "hbm_copy_GBps": round(2 * nbytes / (t_copy / 1e3) / 1e9, 1),
        "hbm_read_GBps": round(nbytes / (t_read / 1e3) / 1e9, 1),
        "hbm_published_GBps": HBM_PEAK_GBS,
        "mfma_bf16_TFLOPs": round(f_mfma / (t_mfma / 1e3) / 1e12, 1),
        "mfma_bf16_published_TFLOPs": PEAK_TFLOPS["bf16"],
        "lds_read_TBps": round(lds_tbs, 2),
        "lds_read_bytes_per_clk_per_cu_at_2.4GHz": round(lds_tbs * 1e12 / (ncu * 2.4e9), 1),
        "compute_units": ncu,
    }


def cold_call_ms(fn, torch, reps=5):
    """Median time of one call right after a 1 GiB device write (which
    evicts x, Psi and the weights from the L2 caches and the MALL)."""
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        flush.fill_(float(len(times)))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del flush
    torch.cuda.empty_cache()
    return round(sorted(times)[len(times) // 2], 4)


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

    from disco_workloads import HEADLINE, WORKLOADS, draw_inputs, round_bf16

    key = args.workload or HEADLINE
    wl = WORKLOADS[key]
    x, w = draw_inputs(wl)
    if wl.dtype == "bf16":
        x, w = round_bf16(x), round_bf16(w)
    # the CPU baseline forks its workers, so it runs before anything
    # initialises the GPU in this process
    cpu = None
    if not args.no_cpu_baseline and not args.fused_only and not args.peaks:
        cpu = cpu_baseline(wl, x, w, args.grid)

    import torch

    import spherical_disco_convolution_amd as sdc

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.peaks:
        print(json.dumps({"measured_peaks": measure_peaks()}), flush=True)
        return

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
    call_s = ev / args.steps
    work = wl.out_points_cout
    value = work / (ms_per_step / 1000.0)

    # the method's algorithmic work per call (the roof definition)
    f_einsum, f_contr = algorithmic_flops(wl, psi.nnz_nonzero)
    f_alg = f_einsum + f_contr
    cig = wl.Ci // wl.groups
    if cig == 1:
        # one input channel per group: weights fold into the taps per channel
        f_folded = 2.0 * wl.B * wl.Co * wl.nlon_out * psi.nnz + 2.0 * wl.Co * psi.nnz_nonzero
        f_alg = min(f_alg, f_folded)
    dsize = 2 if wl.dtype == "bf16" else 4
    peak = PEAK_TFLOPS[wl.dtype]
    bound = "mfma" if wl.dtype == "bf16" else "alu"
    achieved = f_alg / call_s / 1e12
    traffic, traffic_src = measured_traffic(key, "fused_spectral" if spectral else "fused",
                                            args.grid, with_source=True)
    roofline = {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic,
                "traffic_source": traffic_src, "unit_of_work": "one disco_fused_fwd call",
                "call_ms": round(call_s * 1000, 4), "algorithmic_flop": f_alg}

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
    if dom in ("spec_mfma", "spec32_conv"):
        f_dom = spec_mfma_flops(wl, count_windows(psi))
    else:
        f_dom = f_alg
    a_dom = f_dom / dom_s / 1e12
    dominant = {"kernel": dom, "bound": bound, "achieved": round(a_dom, 3), "peak": peak,
                "unit": "TFLOP/s", "frac": round(a_dom / peak, 4),
                "traffic": measured_traffic(key, dom, args.grid), "kernel_ms": round(dom_s * 1000, 4),
                "algorithmic_flop": f_dom}
    extra = {
        "kernels_ms": kernels_ms,
        "dominant_kernel": dominant,
        "algorithmic_bytes": algorithmic_bytes(wl, psi.nnz, dsize),
        "hbm_GBps_algorithmic": round(algorithmic_bytes(wl, psi.nnz, dsize) / call_s / 1e9, 1),
        "psi_build_s": round(psi_build_s, 3),
        "psi_upload_s": round(psi_upload_s, 3),
        "fused_algorithm": "spectral" if spectral else "direct",
    }
    if not args.fused_only:
        extra["cold_ms"] = cold_call_ms(fused, torch)
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
    if not args.no_unfused and not args.fused_only and not args.no_bwd:
        # the fused backward (gradient in the layer's dtype): gx and gw, and
        # gx alone
        gy = torch.randn((wl.B, wl.Co, wl.nlat_out, wl.nlon_out), device="cuda").to(tdt)
        bwd = lambda: sdc.fused_bwd(psi, xd, wd, gy, groups=wl.groups)
        bwd_x = lambda: sdc.fused_bwd(psi, xd, wd, gy, groups=wl.groups, need_gw=False)
        for _ in range(2):
            bwd()
            bwd_x()
        n = 5
        _, t_b = time_region(bwd, n, torch)
        _, t_bx = time_region(bwd_x, n, torch)
        extra["bwd_ms"] = round(t_b / n * 1000, 3)
        extra["bwd_grad_x_ms"] = round(t_bx / n * 1000, 3)
        del gy
    if not args.fused_only and not args.no_peaks:
        extra["measured_peaks"] = measure_peaks()
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
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
