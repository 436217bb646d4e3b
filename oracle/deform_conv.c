/*
 * deform_conv.c -- plain, slow, CPU reference of DeformConv (version 22).
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or constant with the GPU library, and the GPU library never calls it.
 *
 * What it follows ("DeformConv" page, since version 22):
 *   - Inputs: X (N, C, D1..Dn); W (oC, C/group, k1..kn); offset
 *     (N, offset_group * k1*..*kn * n, o1..on), one displacement per kernel
 *     position and spatial axis; optional B (oC); optional mask
 *     (N, offset_group * k1*..*kn, o1..on), default ones.
 *   - Each kernel position samples X at its regular convolution position
 *     plus its offset, by linear interpolation; locations outside the
 *     (padded) input read zero.  The sample is multiplied by the mask, then
 *     by the weight, summed over input channels and kernel positions, plus
 *     the bias.
 *
 * Readings (the page prints no attribute list; its four examples use
 * kernel_shape, pads and offset_group, and fix the rest of the layout):
 *   - offset holds, for kernel position k (row-major over k1..kn) of offset
 *     group g, the n displacements of channels g*K*n + k*n + a, axis a
 *     outermost first (the examples: channel 0 moves tap (0,0) along H,
 *     channel 5 moves tap (1,0) along W);
 *   - input channel c belongs to offset group c / (C / offset_group); the
 *     mask channel of (g, k) is g*K + k;
 *   - strides, dilations, pads (begin values for every axis, then end
 *     values) and group have their convolution meaning: the regular position
 *     of output o and kernel position k along axis a is
 *     o_a * stride_a - pad_begin_a + k_a * dilation_a, and output channel oc
 *     of group G = oc / (oC / group) reads input channels
 *     G*(C/group) .. (G+1)*(C/group)-1 (not exemplified on the page);
 *   - interpolation is linear along every axis with X taken as zero outside
 *     the image (the padded region is zero as well);
 *   - the sampling location (regular position + offset) is computed in the
 *     offset's element type: fp32 for fp32, fp16 and bf16 data (the caller
 *     passes half data widened exactly), float64 for double.  It decides the
 *     taps, so it is computed in that precision; the weights and the sums are
 *     float64.
 */

#include <math.h>
#include <stddef.h>
#include <stdint.h>

/* Every output is computed on its own; a build with -fopenmp splits the
 * output loops over threads without changing any value. */
#ifdef _OPENMP
#define OR_PARALLEL_FOR _Pragma("omp parallel for schedule(dynamic, 256)")
#else
#define OR_PARALLEL_FOR
#endif

#define DC_MAX_RANK 3

/* Linear interpolation of one plane of X (float64, spatial extents in_sp) at
 * the location whose per-axis floor is base and fractional part frac, X zero
 * outside the image: the sum over the 2^r corners, innermost axis fastest, of
 * the product of the per-axis weights (outermost first) times X. */
static double sample_linear(const double *plane, int r, const int64_t *in_sp,
                            const double *frac, const int64_t *base)
{
    double acc = 0.0;
    for (int t = 0; t < (1 << r); ++t) {
        double w = 1.0;
        int valid = 1;
        int64_t off = 0;
        for (int a = 0; a < r; ++a) {
            int bit = (t >> (r - 1 - a)) & 1; /* innermost axis fastest */
            int64_t i = base[a] + bit;
            w *= bit ? frac[a] : 1.0 - frac[a];
            valid = valid && i >= 0 && i < in_sp[a];
            off = off * in_sp[a] + i;
        }
        if (valid)
            acc += w * plane[off];
    }
    return acc;
}

typedef struct {
    const double *X, *Wt, *offset, *B, *mask;
    int r;
    int64_t N, C, OC, og;
    const int64_t *in_sp, *ksz, *out_sp, *strides, *pads, *dilations;
    int64_t Cg, OCg, Cog, K, in_count, out_count;
    int coord_f32;
} dc_problem;

static int dc_setup(dc_problem *P, const double *X, int r, int64_t N, int64_t C,
                    const int64_t *in_sp, const double *Wt, int64_t OC, const int64_t *ksz,
                    const double *offset, const double *B, const double *mask,
                    const int64_t *out_sp, const int64_t *strides, const int64_t *pads,
                    const int64_t *dilations, int64_t group, int64_t offset_group, int coord_f32)
{
    if (r < 1 || r > DC_MAX_RANK || N < 0 || C < 1 || OC < 1 || group < 1 || offset_group < 1)
        return -1;
    if (C % group || OC % group || C % offset_group)
        return -1;
    P->in_count = 1;
    P->out_count = 1;
    P->K = 1;
    for (int a = 0; a < r; ++a) {
        if (in_sp[a] < 1 || ksz[a] < 1 || strides[a] < 1 || dilations[a] < 1 || out_sp[a] < 0)
            return -1;
        int64_t span = dilations[a] * (ksz[a] - 1) + 1;
        int64_t expect = (in_sp[a] + pads[a] + pads[r + a] - span) / strides[a] + 1;
        if (out_sp[a] != expect)
            return -1;
        P->in_count *= in_sp[a];
        P->out_count *= out_sp[a];
        P->K *= ksz[a];
    }
    P->X = X;
    P->Wt = Wt;
    P->offset = offset;
    P->B = B;
    P->mask = mask;
    P->r = r;
    P->N = N;
    P->C = C;
    P->OC = OC;
    P->og = offset_group;
    P->in_sp = in_sp;
    P->ksz = ksz;
    P->out_sp = out_sp;
    P->strides = strides;
    P->pads = pads;
    P->dilations = dilations;
    P->Cg = C / group;
    P->OCg = OC / group;
    P->Cog = C / offset_group;
    P->coord_f32 = coord_f32;
    return 0;
}

/* Output element (n, oc, o): bias + sum over the channels of oc's group and
 * the kernel positions of W * mask * linear sample. */
static double dc_value(const dc_problem *P, int64_t n, int64_t oc, int64_t o)
{
    const int r = P->r;
    const int64_t K = P->K, out_count = P->out_count;
    const int64_t G = oc / P->OCg;
    int64_t oi[DC_MAX_RANK];
    int64_t rest = o;
    for (int a = r - 1; a >= 0; --a) {
        oi[a] = rest % P->out_sp[a];
        rest /= P->out_sp[a];
    }
    double acc = 0.0;
    for (int64_t cl = 0; cl < P->Cg; ++cl) {
        const int64_t c = G * P->Cg + cl;
        const int64_t g = c / P->Cog;
        const double *plane = P->X + (n * P->C + c) * P->in_count;
        for (int64_t k = 0; k < K; ++k) {
            int64_t ki[DC_MAX_RANK];
            int64_t kr = k;
            for (int a = r - 1; a >= 0; --a) {
                ki[a] = kr % P->ksz[a];
                kr /= P->ksz[a];
            }
            double frac[DC_MAX_RANK];
            int64_t base[DC_MAX_RANK];
            int finite = 1;
            for (int a = 0; a < r && finite; ++a) {
                int64_t regular = oi[a] * P->strides[a] - P->pads[a] + ki[a] * P->dilations[a];
                double d = P->offset[((n * P->og + g) * K * r + k * r + a) * out_count + o];
                double loc = P->coord_f32 ? (double)((float)regular + (float)d)
                                          : (double)regular + d;
                /* a location beyond any image reads zero (and is kept away
                 * from the integer conversion) */
                if (!isfinite(loc) || fabs(loc) > 16777216.0) {
                    finite = 0;
                    break;
                }
                double fl = floor(loc); /* exact for an fp32 value too */
                base[a] = (int64_t)fl;
                frac[a] = loc - fl;     /* exact */
            }
            if (!finite)
                continue;
            double v = sample_linear(plane, r, P->in_sp, frac, base);
            if (P->mask)
                v *= P->mask[((n * P->og + g) * K + k) * out_count + o];
            acc += P->Wt[(oc * P->Cg + cl) * K + k] * v;
        }
    }
    if (P->B)
        acc += P->B[oc];
    return acc;
}

/*
 * Y = DeformConv(X, W, offset, B, mask), r spatial axes (1 .. 3).
 *   X      (N, C, in_sp...)            float64
 *   Wt     (OC, C/group, ksz...)       float64
 *   offset (N, og*K*r, out_sp...)      float64 (values of the offset type)
 *   B      (OC) or NULL;  mask (N, og*K, out_sp...) or NULL
 *   strides, dilations: r entries; pads: 2r entries (begins, then ends)
 *   coord_f32: 1 -> locations computed in fp32, 0 -> in float64
 *   Y      (N, OC, out_sp...)          float64, every element written
 * The output extents out_sp are given and must equal
 * (in + pad_begin + pad_end - (dilation * (k - 1) + 1)) / stride + 1.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_deform_conv(const double *X, int r, int64_t N, int64_t C, const int64_t *in_sp,
                       const double *Wt, int64_t OC, const int64_t *ksz, const double *offset,
                       const double *B, const double *mask, const int64_t *out_sp,
                       const int64_t *strides, const int64_t *pads, const int64_t *dilations,
                       int64_t group, int64_t offset_group, int coord_f32, double *Y)
{
    dc_problem P;
    if (dc_setup(&P, X, r, N, C, in_sp, Wt, OC, ksz, offset, B, mask, out_sp, strides, pads,
                 dilations, group, offset_group, coord_f32))
        return -1;
    OR_PARALLEL_FOR
    for (int64_t f = 0; f < N * OC * P.out_count; ++f) {
        const int64_t o = f % P.out_count;
        const int64_t oc = (f / P.out_count) % OC;
        const int64_t n = f / (P.out_count * OC);
        Y[f] = dc_value(&P, n, oc, o);
    }
    return 0;
}

/* As oracle_deform_conv, only for the `count` outputs whose flat indices into
 * Y are listed in `flat`; the values go to Y[0..count).  Returns 0, or -1 on
 * a bad argument or index. */
int oracle_deform_conv_points(const double *X, int r, int64_t N, int64_t C,
                              const int64_t *in_sp, const double *Wt, int64_t OC,
                              const int64_t *ksz, const double *offset, const double *B,
                              const double *mask, const int64_t *out_sp, const int64_t *strides,
                              const int64_t *pads, const int64_t *dilations, int64_t group,
                              int64_t offset_group, int coord_f32, const int64_t *flat,
                              int64_t count, double *Y)
{
    dc_problem P;
    if (dc_setup(&P, X, r, N, C, in_sp, Wt, OC, ksz, offset, B, mask, out_sp, strides, pads,
                 dilations, group, offset_group, coord_f32))
        return -1;
    for (int64_t i = 0; i < count; ++i)
        if (flat[i] < 0 || flat[i] >= N * OC * P.out_count)
            return -1;
    OR_PARALLEL_FOR
    for (int64_t i = 0; i < count; ++i) {
        const int64_t f = flat[i];
        const int64_t o = f % P.out_count;
        const int64_t oc = (f / P.out_count) % OC;
        const int64_t n = f / (P.out_count * OC);
        Y[i] = dc_value(&P, n, oc, o);
    }
    return 0;
}
