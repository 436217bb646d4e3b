// c_abi_check.cpp -- the C ABI of libgsample used from a plain HIP program,
// with no Python and no torch in the process: device memory from hipMalloc,
// the default stream, the HIP runtime of the ROCm install.  It checks
// AffineGrid (bit for bit), GridSample 2-D linear (within 1e-5 of max|X|) and
// nearest (bit for bit after the fp32 rounding), and the fused theta -> sample
// entry point (bit for bit against the unfused pair), each against the oracle
// of this repository (liboracle.so), on seeded inputs.  Exit status 0 when
// every check passes.  Resize (2x bilinear, within 1e-5 of max|X|) and
// DeformConv (fp32 with a workspace, the matrix-core kernel, within 2e-5 of
// the sum of the absolute terms) are checked the same way.  Test
// infrastructure: built next to the tests.
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
int oracle_resize(const float *X, int rank, const int64_t *in_shape, const int64_t *out_shape,
                  const float *scales, int mode, int ct, int nearest_mode, double cubic_a,
                  int exclude_outside, double *Y);
int oracle_deform_conv(const double *X, int r, int64_t N, int64_t C, const int64_t *in_sp,
                       const double *Wt, int64_t OC, const int64_t *ksz, const double *offset,
                       const double *B, const double *mask, const int64_t *out_sp,
                       const int64_t *strides, const int64_t *pads, const int64_t *dilations,
                       int64_t group, int64_t offset_group, int coord_f32, double *Y);
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
    // Resize: 2x bilinear up, half_pixel
    {
        const int64_t ys[4] = {N, C, 2 * H, 2 * W};
        const float sc[4] = {1.0f, 1.0f, 2.0f, 2.0f};
        const size_t nr = (size_t)(N * C * 4 * H * W);
        void *dr = nullptr;
        float *hr = (float *)malloc(nr * 4);
        double *rr = (double *)malloc(nr * 8);
        if (hip_ok(hipMalloc(&dr, nr * 4), "hipMalloc Resize")) {
            expect(gs_resize(dx, GS_F32, xs, 4, ys, sc, GS_RESIZE_LINEAR, GS_CT_HALF_PIXEL,
                             GS_NEAREST_ROUND_PREFER_FLOOR, -0.75f, 0, dr, nullptr) == GS_OK,
                   "gs_resize status");
            hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize");
            hip_ok(hipMemcpy(hr, dr, nr * 4, hipMemcpyDeviceToHost), "hipMemcpy Resize");
            expect(oracle_resize(hx, 4, xs, ys, sc, 1, 0, 0, -0.75, 0, rr) == 0, "oracle_resize");
            double err = 0.0;
            for (size_t i = 0; i < nr; ++i) err = fmax(err, fabs((double)hr[i] - rr[i]));
            printf("resize: max |Y - oracle| = %.3g (bound %.3g)\n", err, 1e-5 * xmax);
            expect(err <= 1e-5 * xmax, "Resize bilinear within 1e-5 max|X| of the oracle");
            hipFree(dr);
        }
        free(hr);
        free(rr);
    }

    // DeformConv, fp32, with a workspace (channels-last copy, matrix cores)
    {
        const int64_t DN = 1, DC = 16, DH = 12, DW = 12, OC = 24, K = 3;
        const int64_t dxs[4] = {DN, DC, DH, DW}, dws[4] = {OC, DC, K, K}, pads[4] = {1, 1, 1, 1};
        const int64_t dsp[2] = {DH, DW}, ksz[2] = {K, K}, ones[2] = {1, 1};
        const size_t nX = (size_t)(DN * DC * DH * DW), nW = (size_t)(OC * DC * K * K),
                     nO = (size_t)(DN * 2 * K * K * DH * DW), nM = (size_t)(DN * K * K * DH * DW),
                     nY = (size_t)(DN * OC * DH * DW);
        float *fX = (float *)malloc(nX * 4), *fW = (float *)malloc(nW * 4), *fO = (float *)malloc(nO * 4);
        float *fM = (float *)malloc(nM * 4), *fB = (float *)malloc(OC * 4), *fY = (float *)malloc(nY * 4);
        double *dX = (double *)malloc(nX * 8), *dWt = (double *)malloc(nW * 8), *dO = (double *)malloc(nO * 8);
        double *dM = (double *)malloc(nM * 8), *dB = (double *)malloc(OC * 8);
        double *ref = (double *)malloc(nY * 8), *S = (double *)malloc(nY * 8);
        for (size_t i = 0; i < nX; ++i) fX[i] = g.next();
        for (size_t i = 0; i < nW; ++i) fW[i] = 0.1f * g.next();
        for (size_t i = 0; i < nO; ++i) fO[i] = 2.0f * g.next();
        for (size_t i = 0; i < nM; ++i) fM[i] = 0.5f * (g.next() + 1.0f);
        for (int64_t i = 0; i < OC; ++i) fB[i] = 0.1f * g.next();
        void *qX = nullptr, *qW = nullptr, *qO = nullptr, *qM = nullptr, *qB = nullptr, *qY = nullptr,
             *qws = nullptr;
        int64_t need = 0;
        expect(gs_deform_conv_workspace_size(GS_F32, dxs, 4, dws, nullptr, pads, nullptr, 1, 1, &need) ==
                       GS_OK && need > 0,
               "gs_deform_conv_workspace_size");
        if (hip_ok(hipMalloc(&qX, nX * 4), "hipMalloc") && hip_ok(hipMalloc(&qW, nW * 4), "hipMalloc") &&
            hip_ok(hipMalloc(&qO, nO * 4), "hipMalloc") && hip_ok(hipMalloc(&qM, nM * 4), "hipMalloc") &&
            hip_ok(hipMalloc(&qB, OC * 4), "hipMalloc") && hip_ok(hipMalloc(&qY, nY * 4), "hipMalloc") &&
            hip_ok(hipMalloc(&qws, (size_t)(need > 0 ? need : 1)), "hipMalloc workspace")) {
            hip_ok(hipMemcpy(qX, fX, nX * 4, hipMemcpyHostToDevice), "hipMemcpy");
            hip_ok(hipMemcpy(qW, fW, nW * 4, hipMemcpyHostToDevice), "hipMemcpy");
            hip_ok(hipMemcpy(qO, fO, nO * 4, hipMemcpyHostToDevice), "hipMemcpy");
            hip_ok(hipMemcpy(qM, fM, nM * 4, hipMemcpyHostToDevice), "hipMemcpy");
            hip_ok(hipMemcpy(qB, fB, OC * 4, hipMemcpyHostToDevice), "hipMemcpy");
            expect(gs_deform_conv(qX, GS_F32, dxs, 4, qW, dws, qO, qB, qM, nullptr, pads, nullptr, 1, 1, qY,
                                  qws, need, nullptr) == GS_OK,
                   "gs_deform_conv status");
            hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize");
            hip_ok(hipMemcpy(fY, qY, nY * 4, hipMemcpyDeviceToHost), "hipMemcpy DeformConv");
            for (size_t i = 0; i < nX; ++i) dX[i] = fX[i];
            for (size_t i = 0; i < nW; ++i) dWt[i] = fW[i];
            for (size_t i = 0; i < nO; ++i) dO[i] = fO[i];
            for (size_t i = 0; i < nM; ++i) dM[i] = fM[i];
            for (int64_t i = 0; i < OC; ++i) dB[i] = fB[i];
            const int64_t st[2] = {1, 1};
            expect(oracle_deform_conv(dX, 2, DN, DC, dsp, dWt, OC, ksz, dO, dB, dM, dsp, st, pads, ones, 1,
                                      1, 1, ref) == 0,
                   "oracle_deform_conv");
            // S: the same sum over the absolute values of X, W, mask and B
            for (size_t i = 0; i < nX; ++i) dX[i] = fabs(dX[i]);
            for (size_t i = 0; i < nW; ++i) dWt[i] = fabs(dWt[i]);
            for (size_t i = 0; i < nM; ++i) dM[i] = fabs(dM[i]);
            for (int64_t i = 0; i < OC; ++i) dB[i] = fabs(dB[i]);
            expect(oracle_deform_conv(dX, 2, DN, DC, dsp, dWt, OC, ksz, dO, dB, dM, dsp, st, pads, ones, 1,
                                      1, 1, S) == 0,
                   "oracle_deform_conv on absolute values");
            double worst = 0.0;
            for (size_t i = 0; i < nY; ++i)
                worst = fmax(worst, fabs((double)fY[i] - ref[i]) / (2e-5 * S[i] + 1e-30));
            printf("deform_conv: max |Y - oracle| / (2e-5 S) = %.3g\n", worst);
            expect(worst <= 1.0, "DeformConv fp32 within 2e-5 of the sum of absolute terms");
        }
        hipFree(qX);
        hipFree(qW);
        hipFree(qO);
        hipFree(qM);
        hipFree(qB);
        hipFree(qY);
        hipFree(qws);
        free(fX); free(fW); free(fO); free(fM); free(fB); free(fY);
        free(dX); free(dWt); free(dO); free(dM); free(dB); free(ref); free(S);
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
