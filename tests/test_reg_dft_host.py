"""The register-resident DFTs of the longitude-spectral kernels, compiled for
the host from the same header (csrc/spectral_dft.h) and compared with the
discrete Fourier transform evaluated from its definition in float64
(tests/host/reg_dft_check.cpp).  The spectral route rests on the DFT over
longitude turning each window's circular correlation into a product per
frequency (DiscreteContinuousConvS2 page, forward equation and the p-shift of
Psi), so a wrong root, sign or index in these templates would break it."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "spherical_disco_convolution_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "host", "reg_dft_check.cpp")


def _compiler():
    return shutil.which("g++")


@pytest.mark.skipif(_compiler() is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_register_dfts_match_float64_definition(tmp_path):
    exe = str(tmp_path / "reg_dft_check")
    subprocess.run([_compiler(), "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__",
                    "-I/opt/rocm/include", "-I" + CSRC, SRC, "-o", exe],
                   check=True, capture_output=True, text=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    seen = set()
    for line in out.strip().splitlines():
        n, s, abs_err, rel_err = line.split()
        n, s, rel_err = int(n), int(s), float(rel_err)
        seen.add((n, s))
        # float32 butterflies: error grows like eps32 * log2(N); 2e-6 is far
        # below what a wrong root or index gives (order 1)
        assert rel_err <= 2e-6, f"reg_dft<{n}, {s}>: relative error {rel_err:.2e}"
    # the lengths the four-step transforms instantiate, both directions
    for n in (4, 8, 16, 45):
        assert (n, -1) in seen and (n, 1) in seen
