/*
 * resize.c -- plain, slow, CPU reference of the Resize operator (version 18)
 * without antialiasing, without region of interest (tf_crop_and_resize).
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or constant with the GPU library, and the GPU library never calls it.
 *
 * What it follows ("Resize" page, version 18):
 *   - Summary: every output value is a weighted average of sampling locations
 *     of the input; output extent = floor(input extent * scale) when scales
 *     are given.
 *   - Attributes: coordinate_transformation_mode (half_pixel,
 *     pytorch_half_pixel, align_corners, asymmetric), mode (nearest, linear,
 *     cubic; linear and cubic are applied axis by axis), nearest_mode (the
 *     four rounding rules), cubic_coeff_a (Keys 1981, Eq. 4),
 *     exclude_outside (zero weight outside the tensor, weights renormalised
 *     to sum 1), keep_aspect_ratio_policy (stretch, not_larger, not_smaller)
 *     and axes.
 *
 * Readings (the page leaves these open; each one agrees with every example
 * the page prints):
 *   - The scale in the coordinate transformation is the value of `scales`
 *     when scales are given, and output extent / input extent when sizes are
 *     given; length_resized is scale * input extent, unfloored, so it equals
 *     the output extent only with sizes (the printed downsample-with-scales
 *     examples, linear and cubic, half_pixel and align_corners, only fit
 *     these values).
 *   - Sampling locations outside the tensor take the value of the nearest
 *     edge element (index clamped), unless exclude_outside is set.
 *   - align_corners with length_resized <= 1 maps to 0, the guard the page
 *     writes for pytorch_half_pixel (it avoids a division by zero).
 *   - The location x_original is computed in fp32, one rounded operation at
 *     a time in the order the page writes the formula (build with
 *     -ffp-contract=off): it decides tap indices, so it is computed in the
 *     element type of the printed examples.  Weights and the sum are float64.
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

#define RZ_MODE_NEAREST 0
#define RZ_MODE_LINEAR 1
#define RZ_MODE_CUBIC 2

#define RZ_CT_HALF_PIXEL 0
#define RZ_CT_PYTORCH_HALF_PIXEL 1
#define RZ_CT_ALIGN_CORNERS 2
#define RZ_CT_ASYMMETRIC 3

#define RZ_NEAREST_ROUND_PREFER_FLOOR 0
#define RZ_NEAREST_ROUND_PREFER_CEIL 1
#define RZ_NEAREST_FLOOR 2
#define RZ_NEAREST_CEIL 3

#define RZ_POLICY_STRETCH 0
#define RZ_POLICY_NOT_LARGER 1
#define RZ_POLICY_NOT_SMALLER 2

#define RZ_MAX_RANK 8

/* Magnitude beyond which a location is clamped before any float->int
 * conversion (only reachable with extreme scales; every such location lies
 * far outside any supported extent, so the clamped tap index is the same).
 * A memory-safety reading; the page says nothing about it. */
#define RZ_COORD_LIMIT 16777216.0f

/* Output extents from scales or sizes (Summary; keep_aspect_ratio_policy).
 * `axes` lists the axes that `values` refer to (count entries); other axes
 * keep their extent.  use_sizes=0: values are scales (float), extent =
 * floor(in * scale), computed in float64 from the fp32 scale.  use_sizes=1:
 * values are sizes; with a policy other than stretch one common scale
 * (min or max over the listed axes of size / extent) gives
 * extent = round-half-up(scale * in).  Returns 0, or -1 on a bad argument. */
int oracle_resize_output_shape(int rank, const int64_t *in_shape, int count, const int64_t *axes,
                               const float *scales, const int64_t *sizes, int use_sizes,
                               int policy, int64_t *out_shape)
{
    if (rank < 1 || rank > RZ_MAX_RANK || count < 0 || count > rank)
        return -1;
    for (int a = 0; a < rank; ++a)
        out_shape[a] = in_shape[a];
    int seen[RZ_MAX_RANK] = {0};
    for (int i = 0; i < count; ++i) {
        int64_t d = axes[i] < 0 ? axes[i] + rank : axes[i];
        if (d < 0 || d >= rank || seen[d])
            return -1;
        seen[d] = 1;
    }
    if (!use_sizes) {
        for (int i = 0; i < count; ++i) {
            int64_t d = axes[i] < 0 ? axes[i] + rank : axes[i];
            if (!(scales[i] > 0.0f))
                return -1;
            out_shape[d] = (int64_t)floor((double)in_shape[d] * (double)scales[i]);
        }
        return 0;
    }
    if (policy == RZ_POLICY_STRETCH) {
        for (int i = 0; i < count; ++i) {
            int64_t d = axes[i] < 0 ? axes[i] + rank : axes[i];
            if (sizes[i] < 0)
                return -1;
            out_shape[d] = sizes[i];
        }
        return 0;
    }
    if (policy != RZ_POLICY_NOT_LARGER && policy != RZ_POLICY_NOT_SMALLER)
        return -1;
    double s = 0.0;
    for (int i = 0; i < count; ++i) {
        int64_t d = axes[i] < 0 ? axes[i] + rank : axes[i];
        if (sizes[i] < 0 || in_shape[d] < 1)
            return -1;
        double r = (double)sizes[i] / (double)in_shape[d];
        if (i == 0 || (policy == RZ_POLICY_NOT_LARGER ? r < s : r > s))
            s = r;
    }
    for (int i = 0; i < count; ++i) {
        int64_t d = axes[i] < 0 ? axes[i] + rank : axes[i];
        out_shape[d] = (int64_t)floor(s * (double)in_shape[d] + 0.5);
    }
    return 0;
}

/* x_original of output index x along an axis (coordinate_transformation_mode).
 * scale and length_resized: see the readings above; n: input extent. */
static float original_coordinate(int64_t x, float scale, float length_resized, int64_t n, int ct)
{
    float xf = (float)x;
    switch (ct) {
    case RZ_CT_HALF_PIXEL:
        return (xf + 0.5f) / scale - 0.5f;
    case RZ_CT_PYTORCH_HALF_PIXEL:
        return length_resized > 1.0f ? (xf + 0.5f) / scale - 0.5f : 0.0f;
    case RZ_CT_ALIGN_CORNERS:
        return length_resized > 1.0f ? xf * (float)(n - 1) / (length_resized - 1.0f) : 0.0f;
    default: /* asymmetric */
        return xf / scale;
    }
}

/* Cubic convolution kernel of Keys (1981, Eq. 4) with coefficient a. */
static double cubic_kernel(double s, double a)
{
    double x = fabs(s);
    if (x <= 1.0)
        return ((a + 2.0) * x - (a + 3.0)) * x * x + 1.0;
    if (x < 2.0)
        return ((a * x - 5.0 * a) * x + 8.0 * a) * x - 4.0 * a;
    return 0.0;
}

typedef struct {
    int count;
    int64_t index[4];
    double weight[4];
} rz_taps;

static int64_t clamp_index(int64_t i, int64_t n)
{
    return i < 0 ? 0 : (i > n - 1 ? n - 1 : i);
}

/* Taps of one axis for location p (fp32) over n input elements. */
static void axis_taps(float p, int64_t n, int mode, int nearest_mode, double a,
                      int exclude_outside, rz_taps *t)
{
    p = p < -RZ_COORD_LIMIT ? -RZ_COORD_LIMIT : (p > RZ_COORD_LIMIT ? RZ_COORD_LIMIT : p);
    if (mode == RZ_MODE_NEAREST) {
        float q;
        switch (nearest_mode) {
        case RZ_NEAREST_ROUND_PREFER_FLOOR: /* halfway cases go down */
            q = ceilf(p - 0.5f);
            break;
        case RZ_NEAREST_ROUND_PREFER_CEIL: /* halfway cases go up */
            q = floorf(p + 0.5f);
            break;
        case RZ_NEAREST_FLOOR:
            q = floorf(p);
            break;
        default:
            q = ceilf(p);
            break;
        }
        t->count = 1;
        t->index[0] = clamp_index((int64_t)q, n);
        t->weight[0] = 1.0;
        return;
    }
    float fl = floorf(p);
    double frac = (double)p - (double)fl; /* exact in float64 */
    int64_t i0 = (int64_t)fl;
    int64_t first;
    if (mode == RZ_MODE_LINEAR) {
        t->count = 2;
        first = i0;
        t->weight[0] = 1.0 - frac;
        t->weight[1] = frac;
    } else {
        t->count = 4;
        first = i0 - 1;
        t->weight[0] = cubic_kernel(frac + 1.0, a);
        t->weight[1] = cubic_kernel(frac, a);
        t->weight[2] = cubic_kernel(1.0 - frac, a);
        t->weight[3] = cubic_kernel(2.0 - frac, a);
    }
    double kept = 0.0;
    for (int j = 0; j < t->count; ++j) {
        int64_t i = first + j;
        if (exclude_outside && (i < 0 || i >= n))
            t->weight[j] = 0.0;
        kept += t->weight[j];
        t->index[j] = clamp_index(i, n);
    }
    if (exclude_outside) {
        for (int j = 0; j < t->count; ++j)
            t->weight[j] = kept != 0.0 ? t->weight[j] / kept : 0.0;
    }
}

typedef struct {
    const float *X;
    int rank;
    const int64_t *in_shape, *out_shape;
    float scale[RZ_MAX_RANK], length_resized[RZ_MAX_RANK];
    int mode, ct, nearest_mode, exclude_outside;
    double cubic_a;
    int64_t out_count;
} rz_problem;

static int rz_setup(rz_problem *P, const float *X, int rank, const int64_t *in_shape,
                    const int64_t *out_shape, const float *scales, int mode, int ct,
                    int nearest_mode, double cubic_a, int exclude_outside)
{
    if (rank < 1 || rank > RZ_MAX_RANK || mode < 0 || mode > 2 || ct < 0 || ct > 3 ||
        nearest_mode < 0 || nearest_mode > 3)
        return -1;
    P->X = X;
    P->rank = rank;
    P->in_shape = in_shape;
    P->out_shape = out_shape;
    P->mode = mode;
    P->ct = ct;
    P->nearest_mode = nearest_mode;
    P->exclude_outside = exclude_outside;
    P->cubic_a = cubic_a;
    P->out_count = 1;
    for (int a = 0; a < rank; ++a) {
        if (in_shape[a] < 0 || out_shape[a] < 0 || (in_shape[a] == 0 && out_shape[a] > 0))
            return -1;
        P->out_count *= out_shape[a];
        if (scales) {
            P->scale[a] = scales[a];
            P->length_resized[a] = (float)in_shape[a] * P->scale[a];
        } else {
            P->scale[a] = in_shape[a] > 0 ? (float)out_shape[a] / (float)in_shape[a] : 1.0f;
            P->length_resized[a] = (float)out_shape[a];
        }
        if (!(P->scale[a] > 0.0f) || !isfinite(P->scale[a]))
            return -1;
    }
    return 0;
}

/* Output element o (flat, row-major): the sum over the product of the
 * per-axis taps of weight * X[taps]. */
static double rz_value(const rz_problem *P, int64_t o)
{
    rz_taps taps[RZ_MAX_RANK];
    int64_t o_idx[RZ_MAX_RANK];
    int64_t rest = o;
    for (int a = P->rank - 1; a >= 0; --a) { /* last axis fastest */
        o_idx[a] = rest % P->out_shape[a];
        rest /= P->out_shape[a];
    }
    for (int a = 0; a < P->rank; ++a) {
        float p = original_coordinate(o_idx[a], P->scale[a], P->length_resized[a],
                                      P->in_shape[a], P->ct);
        axis_taps(p, P->in_shape[a], P->mode, P->nearest_mode, P->cubic_a, P->exclude_outside,
                  &taps[a]);
    }
    int sel[RZ_MAX_RANK] = {0};
    double acc = 0.0;
    for (;;) {
        double w = 1.0;
        int64_t off = 0;
        for (int a = 0; a < P->rank; ++a) {
            w *= taps[a].weight[sel[a]];
            off = off * P->in_shape[a] + taps[a].index[sel[a]];
        }
        acc += w * (double)P->X[off];
        int a = P->rank - 1;
        while (a >= 0) {
            if (++sel[a] < taps[a].count)
                break;
            sel[a] = 0;
            --a;
        }
        if (a < 0)
            break;
    }
    return acc;
}

/*
 * Y = Resize(X): X has `rank` axes with extents in_shape, Y extents
 * out_shape (row-major, float64 output, every element written).
 * scales: per-axis scale (rank entries), length_resized = in_shape[a] * scale
 * in fp32; or NULL (the output extents came from sizes): then the scale of
 * axis a is out_shape[a] / in_shape[a] in fp32 and length_resized is
 * out_shape[a].
 * mode 0 nearest, 1 linear, 2 cubic; ct 0 half_pixel, 1 pytorch_half_pixel,
 * 2 align_corners, 3 asymmetric; nearest_mode 0 round_prefer_floor,
 * 1 round_prefer_ceil, 2 floor, 3 ceil.  Returns 0, or -1 on a bad argument.
 */
int oracle_resize(const float *X, int rank, const int64_t *in_shape, const int64_t *out_shape,
                  const float *scales, int mode, int ct, int nearest_mode, double cubic_a,
                  int exclude_outside, double *Y)
{
    rz_problem P;
    if (rz_setup(&P, X, rank, in_shape, out_shape, scales, mode, ct, nearest_mode, cubic_a,
                 exclude_outside))
        return -1;
    OR_PARALLEL_FOR
    for (int64_t o = 0; o < P.out_count; ++o)
        Y[o] = rz_value(&P, o);
    return 0;
}

/* As oracle_resize, only for the `count` outputs whose flat indices are listed
 * in `flat`; the values go to Y[0..count).  Returns 0, or -1 on a bad argument
 * or index. */
int oracle_resize_points(const float *X, int rank, const int64_t *in_shape,
                         const int64_t *out_shape, const float *scales, int mode, int ct,
                         int nearest_mode, double cubic_a, int exclude_outside,
                         const int64_t *flat, int64_t count, double *Y)
{
    rz_problem P;
    if (rz_setup(&P, X, rank, in_shape, out_shape, scales, mode, ct, nearest_mode, cubic_a,
                 exclude_outside))
        return -1;
    for (int64_t i = 0; i < count; ++i)
        if (flat[i] < 0 || flat[i] >= P.out_count)
            return -1;
    OR_PARALLEL_FOR
    for (int64_t i = 0; i < count; ++i)
        Y[i] = rz_value(&P, flat[i]);
    return 0;
}
