// Host-side check of the Psi builder, the spectral table builder and the
// C-ABI's host paths under AddressSanitizer and UndefinedBehaviorSanitizer.
// Built with g++ -fsanitize=address,undefined from psi_host.cpp,
// spectral_host.cpp, disco_api.cpp and kernel_timing.cpp; the kernel
// launchers and the matrix-core table builder live in the HIP sources and are
// replaced here by stubs that report DISCO_EHIP, so nothing touches a GPU.
// Exit status 0 and the line "asan-driver ok" mean every case ran clean.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "disco_internal.h"

namespace disco {
// stubs for the symbols defined in the HIP sources
static int stub(const char* name) { return set_error(DISCO_EHIP, "%s: not part of the host check", name); }
int launch_contract(const disco_psi*, const void*, int, void*, int, int, int, void*) { return stub("contract"); }
int launch_einsum(const void*, int, const void*, int, const float*, void*, int, int, int, int, int, int,
                  int, int, void*) { return stub("einsum"); }
int launch_fused(const disco_psi*, const void*, int, const void*, const float*, void*, int, int, int,
                 int, int, void*) { return stub("fused"); }
int launch_fused_noalloc(const disco_psi*, const void*, int, const void*, const float*, void*, int, int,
                         int, int, int, void*) { return stub("fused_noalloc"); }
int fused_spectral_eligible(const disco_psi*, int, int, int, int) { return 0; }
int launch_fill_zero(float*, size_t, void*) { return stub("fill_zero"); }
int launch_contract_transpose(const disco_psi*, const void*, int, void*, int, int, int, void*) {
    return stub("contract_transpose");
}
int launch_einsum_grad_xk(const void*, int, const void*, int, void*, int, int, int, int, int, int, int,
                          int, void*) { return stub("grad_xk"); }
int launch_einsum_grad_w(const void*, int, const void*, int, float*, int, int, int, int, int, int, int,
                         void*) { return stub("grad_w"); }
int launch_fused_bwd(const disco_psi*, const void*, int, const void*, int, const void*, int, void*, int,
                     float*, float*, int, int, int, int, void*) { return stub("fused_bwd"); }
int build_mfma_tables(disco_psi*, std::vector<char>&, std::vector<int32_t>&) { return DISCO_OK; }
}  // namespace disco

static int g_fail = 0;
#define CHECK(c)                                                                       \
    do {                                                                               \
        if (!(c)) {                                                                    \
            std::printf("FAIL %s:%d %s (%s)\n", __FILE__, __LINE__, #c, disco_last_error()); \
            ++g_fail;                                                                  \
        }                                                                              \
    } while (0)

static disco_psi_desc desc(int nli, int nlo_i, int nlo, int nlo_o, int nr, int nphi, double tc,
                           int grid = DISCO_GRID_EQUIANGULAR) {
    disco_psi_desc d{};
    d.nlat_in = nli;
    d.nlon_in = nlo_i;
    d.nlat_out = nlo;
    d.nlon_out = nlo_o;
    d.grid_in = d.grid_out = grid;
    d.basis_type = DISCO_BASIS_PIECEWISE_LINEAR;
    d.basis_norm = DISCO_NORM_NONE;
    d.kernel_shape[0] = nr;
    d.kernel_shape[1] = nphi;
    d.theta_cutoff = tc;
    return d;
}

// build, query, export into exactly sized buffers, build the spectral tables,
// try the upload (no GPU here: an error, not a crash), free
static void run_valid(const disco_psi_desc& d) {
    disco_psi* psi = nullptr;
    CHECK(disco_psi_build(&d, &psi) == DISCO_OK);
    if (!psi) return;
    int32_t K = 0;
    int64_t nnz = 0, nz = 0;
    double tc = 0.0;
    CHECK(disco_psi_query(psi, &K, &nnz, &nz, &tc) == DISCO_OK);
    CHECK(K >= 1 && nnz > 0 && nz > 0 && nz <= nnz * K && tc > 0.0);
    std::vector<int64_t> row_ptr(d.nlat_out + 1);
    std::vector<int32_t> in_lat(nnz), lon_off(nnz);
    std::vector<double> vals((size_t)nnz * K);
    CHECK(disco_psi_export(psi, row_ptr.data(), in_lat.data(), lon_off.data(), vals.data()) == DISCO_OK);
    CHECK(row_ptr[0] == 0 && row_ptr[d.nlat_out] == nnz);
    for (int64_t n = 0; n < nnz; ++n) {
        CHECK(in_lat[n] >= 0 && in_lat[n] < d.nlat_in);
        CHECK(lon_off[n] >= 0 && lon_off[n] < d.nlon_in);
        if (g_fail) break;
    }
    std::vector<uint32_t> psih;
    std::vector<float> psih32;
    int32_t radix[disco::kSpecMaxRadix] = {0}, nrad = 0, mp = 0;
    CHECK(disco::build_spectral_tables(psi->host, psih, psih32, radix, &nrad, &mp) == DISCO_OK);
    if (mp > 0) {
        CHECK(psih.size() >= (size_t)psi->host.windows.size() * K * mp);
        for (size_t n = 0; n < psih32.size(); ++n)
            if (!std::isfinite(psih32[n])) { CHECK(!"non-finite Psi_hat"); break; }
    }
    // without a GPU the upload must fail cleanly
    const int rc = disco_psi_to_device(psi);
    CHECK(rc == DISCO_OK || rc == DISCO_EHIP);
    disco_psi_free(psi);
}

static void run_invalid(const disco_psi_desc& d, int expect) {
    disco_psi* psi = reinterpret_cast<disco_psi*>(0x1);
    const int rc = disco_psi_build(&d, &psi);
    CHECK(rc == expect);
    CHECK(psi == nullptr);
    CHECK(disco_last_error()[0] != '\0');
}

int main() {
    const double pi = 3.14159265358979323846;
    // the five workload shapes' small relatives and the edge cases of the builder
    run_valid(desc(33, 64, 33, 64, 3, 0, 4 * pi / 32));                 // isotropic, stride 1
    run_valid(desc(65, 128, 65, 128, 3, 3, 4 * pi / 64));               // anisotropic, K = 7
    run_valid(desc(61, 120, 31, 60, 3, 3, 4 * pi / 30));                // stride 2, halved latitude
    run_valid(desc(41, 80, 21, 40, 5, 4, 6 * pi / 20));                 // K = 17, stride 2
    run_valid(desc(17, 32, 17, 32, 2, 1, 0.0));                         // nphi = 1, default cutoff
    run_valid(desc(9, 12, 9, 12, 3, 3, 3.0));                           // full-ring windows
    run_valid(desc(5, 1, 5, 1, 1, 0, 1.0));                             // one longitude
    run_valid(desc(2, 8, 2, 8, 1, 0, 0.5));                             // two latitudes (poles only)
    run_valid(desc(33, 64, 17, 16, 3, 3, 4 * pi / 16));                 // stride 4
    for (int g = DISCO_GRID_LEGENDRE_GAUSS; g <= DISCO_GRID_EQUIANGULAR_TRAPEZOIDAL; ++g)
        run_valid(desc(32, 64, 32, 64, 3, 3, 4 * pi / 31, g));
    // argument errors: reported, nothing built
    run_invalid(desc(33, 64, 33, 48, 3, 0, 0.3), DISCO_EINVAL);          // non-integer stride
    run_invalid(desc(1, 64, 33, 64, 3, 0, 0.3), DISCO_EINVAL);           // one latitude
    run_invalid(desc(33, 64, 33, 64, 0, 0, 0.3), DISCO_EINVAL);          // nr = 0
    run_invalid(desc(33, 64, 33, 64, 3, -1, 0.3), DISCO_EINVAL);         // nphi < 0
    run_invalid(desc(33, 64, 33, 64, 3, 0, pi), DISCO_EINVAL);           // cutoff = pi
    run_invalid(desc(33, 64, 33, 64, 3, 0, std::nan("")), DISCO_EINVAL); // NaN cutoff
    run_invalid(desc(33, 64, 33, 64, 3, 0, 0.3, 7), DISCO_EUNSUPPORTED); // unknown grid
    {
        disco_psi_desc d = desc(33, 64, 33, 64, 3, 0, 0.3);
        d.basis_norm = 1;
        run_invalid(d, DISCO_EUNSUPPORTED);
    }
    CHECK(disco_psi_build(nullptr, nullptr) == DISCO_EINVAL);
    CHECK(disco_psi_query(nullptr, nullptr, nullptr, nullptr, nullptr) == DISCO_EINVAL);
    CHECK(disco_psi_export(nullptr, nullptr, nullptr, nullptr, nullptr) == DISCO_EINVAL);
    disco_psi_free(nullptr);
    // compute calls with NULL arguments fail before any launch
    CHECK(disco_contract(nullptr, nullptr, DISCO_F32, nullptr, DISCO_F32, 1, 1, nullptr) == DISCO_EINVAL);
    CHECK(disco_fused_fwd(nullptr, nullptr, DISCO_F32, nullptr, DISCO_F32, nullptr, nullptr, DISCO_F32, 1,
                          1, 1, 1, nullptr) == DISCO_EINVAL);
    if (g_fail) {
        std::printf("asan-driver: %d failures\n", g_fail);
        return 1;
    }
    std::printf("asan-driver ok\n");
    return 0;
}
