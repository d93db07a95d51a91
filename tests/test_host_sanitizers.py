"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer: the Psi
builder (psi_host.cpp), the spectral table builder (spectral_host.cpp) and the
C-ABI's host paths (disco_api.cpp, kernel_timing.cpp), built with g++ and
driven by tests/host/asan_driver.cpp over the builder's edge cases (strides 1,
2 and 4, K = 1..17, full-ring windows, one longitude, two latitudes, every
latitude grid) and its argument errors.  Exactly sized export buffers let the
sanitizer catch any write past what disco_psi_query reports.  No GPU is
touched: the kernel launchers are stubs in the driver."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "spherical_disco_convolution_amd", "csrc")
HOST_SOURCES = ["psi_host.cpp", "spectral_host.cpp", "disco_api.cpp", "kernel_timing.cpp"]


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/lib"),
                    reason="needs g++ and the ROCm runtime library")
def test_host_code_is_sanitizer_clean(tmp_path):
    flags = ["-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
             "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
             "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
    objs = []
    for src in HOST_SOURCES:
        obj = str(tmp_path / (src + ".o"))
        r = subprocess.run(["g++", "-c"] + flags + [os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    exe = str(tmp_path / "asan_driver")
    r = subprocess.run(["g++"] + flags + [os.path.join(ROOT, "tests", "host", "asan_driver.cpp")] +
                       objs + ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                               "-lpthread", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0 and "asan-driver ok" in r.stdout, report[-4000:]
    assert "runtime error" not in report, report[-4000:]
