// c_abi_check.cpp -- the C ABI of libgsample used from a plain HIP program,
// with no Python and no torch in the process: device memory from hipMalloc,
// the default stream, the HIP runtime of the ROCm install.  It checks
// AffineGrid (bit for bit), GridSample 2-D linear (within 1e-5 of max|X|) and
// nearest (bit for bit after the fp32 rounding), and the fused theta -> sample
// entry point (bit for bit against the unfused pair), each against the oracle
// of this repository (liboracle.so), on seeded inputs.  Exit status 0 when
// every check passes.  Test infrastructure: built next to the tests.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gsample.h"

extern "C" {
int oracle_affine_grid(const float *theta, int r, int64_t N, const int64_t *out_spatial,
                       int align_corners, float *grid);
int oracle_grid_sample(const float *X, int r, int64_t N, int64_t C, const int64_t *in_spatial,
                       const float *grid, const int64_t *out_spatial, int mode, int padding,
                       int align_corners, double *Y);
}

namespace {

// 64-bit linear congruential generator (Knuth's MMIX constants), top 24 bits
// as a float in [-1, 1).
struct Lcg {
    uint64_t s;
    float next() {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        return (float)((int32_t)(s >> 40) - (1 << 23)) / (float)(1 << 23);
    }
};

int failures = 0;

void expect(bool ok, const char *what) {
    printf("%s: %s\n", ok ? "ok" : "FAILED", what);
    if (!ok) ++failures;
}

bool hip_ok(hipError_t e, const char *where) {
    if (e != hipSuccess) {
        printf("FAILED: %s: %s\n", where, hipGetErrorString(e));
        ++failures;
        return false;
    }
    return true;
}

}  // namespace

int main() {
    int rt = 0;
    hipRuntimeGetVersion(&rt);
    printf("HIP runtime %d, libgsample ABI %d\n", rt, gs_abi_version());

    const int64_t N = 2, C = 3, H = 20, W = 24, OH = 13, OW = 17;
    const int64_t xs[4] = {N, C, H, W}, size[4] = {N, C, OH, OW}, gs_shape[4] = {N, OH, OW, 2};
    const int64_t in_sp[2] = {H, W}, out_sp[2] = {OH, OW};
    const size_t nx = (size_t)(N * C * H * W), ng = (size_t)(N * OH * OW * 2),
                 ny = (size_t)(N * C * OH * OW);
    float *hx = (float *)malloc(nx * 4), *htheta = (float *)malloc(N * 6 * 4);
    float *hgrid = (float *)malloc(ng * 4), *rgrid = (float *)malloc(ng * 4);
    float *hy = (float *)malloc(ny * 4), *hyf = (float *)malloc(ny * 4);
    double *ry = (double *)malloc(ny * 8);
    Lcg g{12345};
    for (size_t i = 0; i < nx; ++i) hx[i] = g.next();
    for (int64_t n = 0; n < N; ++n)
        for (int k = 0; k < 6; ++k)
            htheta[n * 6 + k] = (k == 0 || k == 4 ? 1.0f : 0.0f) + 0.2f * g.next();
    float xmax = 0.0f;
    for (size_t i = 0; i < nx; ++i) xmax = fmaxf(xmax, fabsf(hx[i]));

    void *dx = nullptr, *dtheta = nullptr, *dgrid = nullptr, *dy = nullptr, *dyf = nullptr;
    if (!hip_ok(hipMalloc(&dx, nx * 4), "hipMalloc") || !hip_ok(hipMalloc(&dtheta, N * 6 * 4), "hipMalloc") ||
        !hip_ok(hipMalloc(&dgrid, ng * 4), "hipMalloc") || !hip_ok(hipMalloc(&dy, ny * 4), "hipMalloc") ||
        !hip_ok(hipMalloc(&dyf, ny * 4), "hipMalloc"))
        return 1;
    hip_ok(hipMemcpy(dx, hx, nx * 4, hipMemcpyHostToDevice), "hipMemcpy X");
    hip_ok(hipMemcpy(dtheta, htheta, N * 6 * 4, hipMemcpyHostToDevice), "hipMemcpy theta");

    // AffineGrid
    expect(gs_affine_grid(dtheta, GS_F32, size, 4, 0, dgrid, nullptr) == GS_OK, "gs_affine_grid status");
    hip_ok(hipMemcpy(hgrid, dgrid, ng * 4, hipMemcpyDeviceToHost), "hipMemcpy grid");
    expect(oracle_affine_grid(htheta, 2, N, out_sp, 0, rgrid) == 0, "oracle_affine_grid");
    expect(memcmp(hgrid, rgrid, ng * 4) == 0, "AffineGrid equals the oracle bit for bit");

    for (int mode : {(int)GS_MODE_LINEAR, (int)GS_MODE_NEAREST}) {
        const bool lin = mode == GS_MODE_LINEAR;
        expect(gs_grid_sample_2d(dx, GS_F32, xs, dgrid, GS_F32, gs_shape, mode, GS_PAD_ZEROS, 0, dy,
                                 nullptr) == GS_OK,
               lin ? "gs_grid_sample_2d linear status" : "gs_grid_sample_2d nearest status");
        expect(gs_affine_grid_sample_fused(dtheta, GS_F32, dx, GS_F32, xs, 4, out_sp, mode, GS_PAD_ZEROS, 0,
                                           dyf, nullptr) == GS_OK,
               "gs_affine_grid_sample_fused status");
        hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize");
        hip_ok(hipMemcpy(hy, dy, ny * 4, hipMemcpyDeviceToHost), "hipMemcpy Y");
        hip_ok(hipMemcpy(hyf, dyf, ny * 4, hipMemcpyDeviceToHost), "hipMemcpy Y fused");
        expect(oracle_grid_sample(hx, 2, N, C, in_sp, rgrid, out_sp, mode, 0, 0, ry) == 0,
               "oracle_grid_sample");
        double err = 0.0;
        size_t exact = 0;
        for (size_t i = 0; i < ny; ++i) {
            err = fmax(err, fabs((double)hy[i] - ry[i]));
            exact += hy[i] == (float)ry[i];
        }
        if (lin) {
            printf("linear: max |Y - oracle| = %.3g (bound %.3g)\n", err, 1e-5 * xmax);
            expect(err <= 1e-5 * xmax, "GridSample linear within 1e-5 max|X| of the oracle");
        } else {
            expect(exact == ny, "GridSample nearest equals the oracle bit for bit");
        }
        expect(memcmp(hy, hyf, ny * 4) == 0, "fused equals AffineGrid then GridSample bit for bit");
    }
    hipFree(dx);
    hipFree(dtheta);
    hipFree(dgrid);
    hipFree(dy);
    hipFree(dyf);
    free(hx);
    free(htheta);
    free(hgrid);
    free(rgrid);
    free(hy);
    free(hyf);
    free(ry);
    if (failures)
        printf("c abi check FAILED (%d)\n", failures);
    else
        printf("c abi check ok\n");
    return failures ? 1 : 0;
}
