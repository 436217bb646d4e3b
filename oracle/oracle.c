/*
 * oracle.c -- plain, slow, CPU reference of the spatial-transformer grid
 * generator (AffineGrid) and sampler (GridSample).
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or constant with the GPU library, and the GPU library never calls it.
 *
 * What it follows (ONNX operator pages):
 *   - "AffineGrid" (since version 20): Summary (homogeneous affine matrix,
 *     implicit last row, evenly spaced positions over [-1, 1], the meaning of
 *     align_corners), Inputs (theta, size), Outputs (grid).
 *   - "GridSample - version 20": Summary (shapes, pixel-centre convention,
 *     innermost-first order of the location vector), Attributes
 *     (align_corners, mode, padding_mode).
 *   - "GridSample" (version 22): same definition, bfloat16 added to the types.
 *   - "Resize" (version 18), Attributes: cubic_coeff_a, whose default -0.75
 *     is the coefficient of the cubic convolution kernel of Keys (1981,
 *     Eq. 4) that the page refers to.
 *
 * Precision (the readings behind these choices are listed with the design
 * notes of the repository):
 *   - Grid generation and un-normalisation are carried out in the grid's own
 *     element type, one rounded operation at a time, in the order written
 *     below (build with -ffp-contract=off): fp32 for fp32 grids (the type of
 *     every grid on the pages; fp16 / bf16 grids are widened exactly to fp32
 *     first), float64 for double grids.  These steps decide integer tap
 *     indices.
 *   - Interpolation weights and the weighted sum are carried out in float64
 *     and returned unrounded; X may be given as fp32 or as float64 (double X,
 *     and integer X converted to float64: the GridSample page computes
 *     integer inputs in floating point and casts at the end, a cast the
 *     Python side of the oracle applies).
 *
 * What pins it (tests/test_oracle_*.py): the worked examples printed on the
 * AffineGrid and GridSample pages, the Resize cubic and linear examples
 * re-expressed as border-padded sampling, closed forms (identity transform,
 * constant input, affine ramps, symmetry and periodicity of reflection), a
 * dense-lattice brute force on tiny inputs with numpy's padding modes, and the
 * torch CPU functions the pages name under "See also".
 *
 * Non-finite locations (the pages are silent): the output is 0 for every
 * channel.  This is a memory-safety reading, not a value the pages fix.
 */

#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* Every output is computed on its own.  A build with -fopenmp (used to time
 * the oracle on all host cores, and for large parity checks) splits the
 * output loops over threads; each output still runs the same code, so the
 * values do not depend on the thread count.  Without -fopenmp the loops are
 * serial. */
#ifdef _OPENMP
#include <omp.h>
#define OR_PARALLEL_FOR _Pragma("omp parallel for schedule(dynamic, 256)")
#else
#define OR_PARALLEL_FOR
#endif

#define OR_MODE_LINEAR 0
#define OR_MODE_NEAREST 1
#define OR_MODE_CUBIC 2

#define OR_PAD_ZEROS 0
#define OR_PAD_BORDER 1
#define OR_PAD_REFLECTION 2

#define OR_MAX_RANK 8

/* Magnitude beyond which a coordinate is clamped before any float->int
 * conversion.  Every such coordinate lies far outside any supported extent, or
 * carries no fractional bits; the pages say nothing about it (memory-safety
 * reading only). */
#define OR_COORD_LIMIT 16777216.0f

int oracle_abi_version(void) { return 1; }

/* Threads the output loops use: 1 unless built with -fopenmp. */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int oracle_grid_sample_ex(const float *X, const double *Xd, int r, int64_t N, int64_t C,
                          const int64_t *in_spatial, const float *grid, const double *gridd,
                          const int64_t *out_spatial, int mode, int padding, int align_corners,
                          double *Y);
int oracle_grid_sample_points_ex(const float *X, const double *Xd, int r, int64_t N, int64_t C,
                                 const int64_t *in_spatial, const float *grid,
                                 const double *gridd, const int64_t *out_spatial, int mode,
                                 int padding, int align_corners, const int64_t *flat,
                                 int64_t count, double *Y);

/* ---------------------------------------------------------------------- */
/* AffineGrid                                                              */
/* ---------------------------------------------------------------------- */

/* Position of sample i of m evenly spaced samples over [-1, 1].
 * align_corners=1: -1 and 1 are the centres of the first and last pixel, so
 * the samples are -1 + 2i/(m-1).  A single sample sits at the centre, 0.
 * align_corners=0: -1 and 1 are the outer edges of the corner pixels, so the
 * samples are the pixel centres -1 + (2i+1)/m. */
static float base_position(int64_t i, int64_t m, int align_corners)
{
    if (align_corners) {
        if (m == 1)
            return 0.0f;
        return (float)(2 * i) / (float)(m - 1) - 1.0f;
    }
    return (float)(2 * i + 1) / (float)m - 1.0f;
}

/*
 * grid[n, o_0, ..., o_{r-1}, k] = sum_j theta[n, k, j] * b_j + theta[n, k, r]
 *
 * theta: (N, r, r+1) fp32, row k produces component k of the output vector.
 * out_spatial: r extents, outermost first ((H, W) or (D, H, W)).
 * The position vector b is listed innermost axis first: b_0 runs along the
 * last spatial axis (W), b_1 along the one before (H), b_2 along D.  Each
 * product and sum is rounded to fp32, summed left to right, translation last.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_affine_grid(const float *theta, int r, int64_t N, const int64_t *out_spatial,
                       int align_corners, float *grid)
{
    if (r < 1 || r > OR_MAX_RANK || N < 0)
        return -1;
    int64_t count = 1;
    for (int a = 0; a < r; ++a) {
        if (out_spatial[a] < 0)
            return -1;
        count *= out_spatial[a];
    }
    OR_PARALLEL_FOR
    for (int64_t nf = 0; nf < N * count; ++nf) {
        const int64_t n = nf / count, flat = nf % count;
        const float *th = theta + n * r * (r + 1);
        {
            /* split the flat location into per-axis indices (outermost first) */
            int64_t idx[OR_MAX_RANK];
            int64_t rem = flat;
            for (int a = r - 1; a >= 0; --a) {
                idx[a] = rem % out_spatial[a];
                rem /= out_spatial[a];
            }
            float b[OR_MAX_RANK]; /* innermost first */
            for (int j = 0; j < r; ++j) {
                int a = r - 1 - j;
                b[j] = base_position(idx[a], out_spatial[a], align_corners);
            }
            float *out = grid + (n * count + flat) * r;
            for (int k = 0; k < r; ++k) {
                const float *row = th + k * (r + 1);
                float s = row[0] * b[0];
                for (int j = 1; j < r; ++j) {
                    float prod = row[j] * b[j];
                    s = s + prod;
                }
                s = s + row[r];
                out[k] = s;
            }
        }
    }
    return 0;
}

/* AffineGrid with a double theta: the same steps in float64 (the grid is
 * double too; AffineGrid page, Type Constraints: theta and grid share T1). */
static double base_position_d(int64_t i, int64_t m, int align_corners)
{
    if (align_corners) {
        if (m == 1)
            return 0.0;
        return (double)(2 * i) / (double)(m - 1) - 1.0;
    }
    return (double)(2 * i + 1) / (double)m - 1.0;
}

int oracle_affine_grid_d(const double *theta, int r, int64_t N, const int64_t *out_spatial,
                         int align_corners, double *grid)
{
    if (r < 1 || r > OR_MAX_RANK || N < 0)
        return -1;
    int64_t count = 1;
    for (int a = 0; a < r; ++a) {
        if (out_spatial[a] < 0)
            return -1;
        count *= out_spatial[a];
    }
    OR_PARALLEL_FOR
    for (int64_t nf = 0; nf < N * count; ++nf) {
        const int64_t n = nf / count, flat = nf % count;
        const double *th = theta + n * r * (r + 1);
        {
            int64_t idx[OR_MAX_RANK];
            int64_t rem = flat;
            for (int a = r - 1; a >= 0; --a) {
                idx[a] = rem % out_spatial[a];
                rem /= out_spatial[a];
            }
            double b[OR_MAX_RANK]; /* innermost first */
            for (int j = 0; j < r; ++j) {
                int a = r - 1 - j;
                b[j] = base_position_d(idx[a], out_spatial[a], align_corners);
            }
            double *out = grid + (n * count + flat) * r;
            for (int k = 0; k < r; ++k) {
                const double *row = th + k * (r + 1);
                double s = row[0] * b[0];
                for (int j = 1; j < r; ++j) {
                    double prod = row[j] * b[j];
                    s = s + prod;
                }
                s = s + row[r];
                out[k] = s;
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* GridSample                                                              */
/* ---------------------------------------------------------------------- */

/* Normalised location g in [-1, 1] -> pixel coordinate along an axis of
 * extent n.  align_corners=1: -1 and 1 are the centres of pixels 0 and n-1.
 * align_corners=0: -1 and 1 are the outer edges of those pixels, i.e. pixel
 * coordinates -0.5 and n-0.5. */
static float unnormalize(float g, int64_t n, int align_corners)
{
    if (align_corners) {
        float u = (g + 1.0f) / 2.0f;
        return u * (float)(n - 1);
    }
    float v = (g + 1.0f) * (float)n;
    return (v - 1.0f) / 2.0f;
}

/* Fold p into [lo, hi] by repeated reflection at the two borders. */
static float reflect(float p, float lo, float hi)
{
    float span = hi - lo;
    if (span <= 0.0f)
        return 0.0f;
    float d = fabsf(p - lo);
    float f = floorf(d / span);
    float fs = f * span;
    float e = d - fs;
    float half = floorf(f * 0.5f);
    int odd = (f - 2.0f * half) != 0.0f;
    return odd ? hi - e : lo + e;
}

static float clampf(float v, float lo, float hi)
{
    return v < lo ? lo : (v > hi ? hi : v);
}

static void reflect_bounds(int64_t n, int align_corners, float *lo, float *hi)
{
    if (align_corners) {
        *lo = 0.0f;
        *hi = (float)(n - 1);
    } else {
        *lo = -0.5f;
        *hi = (float)n - 0.5f;
    }
}

/* Coordinate padding used by nearest and linear: border clamps the location
 * into the image; reflection folds it at the borders and then clamps (the
 * fold can leave it up to half a pixel outside when align_corners=0). */
static float pad_coordinate(float p, int64_t n, int padding, int align_corners)
{
    if (padding == OR_PAD_BORDER)
        return clampf(p, 0.0f, (float)(n - 1));
    if (padding == OR_PAD_REFLECTION) {
        float lo, hi;
        reflect_bounds(n, align_corners, &lo, &hi);
        return clampf(reflect(p, lo, hi), 0.0f, (float)(n - 1));
    }
    return p;
}

/* Rounding half to even (the nearest-mode rule of the GridSample page);
 * rintf rounds ties to even in the default rounding mode. */
static int64_t round_half_even(float p)
{
    return (int64_t)rintf(p);
}

/* Cubic convolution kernel of Keys (1981, Eq. 4) with coefficient a. */
static double keys_kernel(double s, double a)
{
    double x = fabs(s);
    if (x <= 1.0)
        return ((a + 2.0) * x - (a + 3.0)) * x * x + 1.0;
    if (x < 2.0)
        return ((a * x - 5.0 * a) * x + 8.0 * a) * x - 4.0 * a;
    return 0.0;
}

#define OR_CUBIC_A (-0.75)

/* The same coordinate steps for a double grid, in float64 (one rounded
 * operation at a time, same order and bounds as the fp32 functions above). */
static double unnormalize_d(double g, int64_t n, int align_corners)
{
    if (align_corners) {
        double u = (g + 1.0) / 2.0;
        return u * (double)(n - 1);
    }
    double v = (g + 1.0) * (double)n;
    return (v - 1.0) / 2.0;
}

static double reflect_d(double p, double lo, double hi)
{
    double span = hi - lo;
    if (span <= 0.0)
        return 0.0;
    double d = fabs(p - lo);
    double f = floor(d / span);
    double fs = f * span;
    double e = d - fs;
    double half = floor(f * 0.5);
    int odd = (f - 2.0 * half) != 0.0;
    return odd ? hi - e : lo + e;
}

static double clamp_d(double v, double lo, double hi)
{
    return v < lo ? lo : (v > hi ? hi : v);
}

static void reflect_bounds_d(int64_t n, int align_corners, double *lo, double *hi)
{
    if (align_corners) {
        *lo = 0.0;
        *hi = (double)(n - 1);
    } else {
        *lo = -0.5;
        *hi = (double)n - 0.5;
    }
}

static double pad_coordinate_d(double p, int64_t n, int padding, int align_corners)
{
    if (padding == OR_PAD_BORDER)
        return clamp_d(p, 0.0, (double)(n - 1));
    if (padding == OR_PAD_REFLECTION) {
        double lo, hi;
        reflect_bounds_d(n, align_corners, &lo, &hi);
        return clamp_d(reflect_d(p, lo, hi), 0.0, (double)(n - 1));
    }
    return p;
}

/* Per-axis taps of one location: up to 4 (index, weight, valid) triples. */
typedef struct {
    int count;
    int64_t index[4];
    double weight[4];
    int valid[4];
} axis_taps;

/* Taps along one axis of extent n for location g; returns 0 if the location
 * is not finite (then the output is 0 for every channel). */
static int make_axis_taps(float g, int64_t n, int mode, int padding, int align_corners,
                          axis_taps *t)
{
    float p = unnormalize(g, n, align_corners);
    if (!isfinite(p))
        return 0;
    p = clampf(p, -OR_COORD_LIMIT, OR_COORD_LIMIT);

    if (mode == OR_MODE_NEAREST) {
        float q = pad_coordinate(p, n, padding, align_corners);
        int64_t i = round_half_even(q);
        t->count = 1;
        t->index[0] = i;
        t->weight[0] = 1.0;
        t->valid[0] = (i >= 0 && i < n);
        return 1;
    }

    if (mode == OR_MODE_LINEAR) {
        float q = pad_coordinate(p, n, padding, align_corners);
        float fl = floorf(q);
        double frac = (double)q - (double)fl; /* exact in float64 */
        int64_t i0 = (int64_t)fl;
        t->count = 2;
        t->index[0] = i0;
        t->index[1] = i0 + 1;
        t->weight[0] = 1.0 - frac;
        t->weight[1] = frac;
        for (int j = 0; j < 2; ++j)
            t->valid[j] = (t->index[j] >= 0 && t->index[j] < n);
        return 1;
    }

    /* cubic: the location itself is not padded; each of the four taps is. */
    float fl = floorf(p);
    double frac = (double)p - (double)fl;
    int64_t i0 = (int64_t)fl;
    t->count = 4;
    t->weight[0] = keys_kernel(frac + 1.0, OR_CUBIC_A);
    t->weight[1] = keys_kernel(frac, OR_CUBIC_A);
    t->weight[2] = keys_kernel(1.0 - frac, OR_CUBIC_A);
    t->weight[3] = keys_kernel(2.0 - frac, OR_CUBIC_A);
    for (int j = 0; j < 4; ++j) {
        int64_t i = i0 - 1 + j;
        if (padding == OR_PAD_ZEROS) {
            t->index[j] = i;
            t->valid[j] = (i >= 0 && i < n);
        } else if (padding == OR_PAD_BORDER) {
            t->index[j] = i < 0 ? 0 : (i > n - 1 ? n - 1 : i);
            t->valid[j] = 1;
        } else {
            float lo, hi;
            reflect_bounds(n, align_corners, &lo, &hi);
            float q = clampf(reflect((float)i, lo, hi), 0.0f, (float)(n - 1));
            t->index[j] = (int64_t)q;
            t->valid[j] = 1;
        }
    }
    return 1;
}

/* make_axis_taps for a location of a double grid: the coordinate steps in
 * float64, the taps and weights as above. */
static int make_axis_taps_d(double g, int64_t n, int mode, int padding, int align_corners,
                            axis_taps *t)
{
    double p = unnormalize_d(g, n, align_corners);
    if (!isfinite(p))
        return 0;
    p = clamp_d(p, -(double)OR_COORD_LIMIT, (double)OR_COORD_LIMIT);

    if (mode == OR_MODE_NEAREST) {
        double q = pad_coordinate_d(p, n, padding, align_corners);
        int64_t i = (int64_t)rint(q); /* ties to even */
        t->count = 1;
        t->index[0] = i;
        t->weight[0] = 1.0;
        t->valid[0] = (i >= 0 && i < n);
        return 1;
    }

    if (mode == OR_MODE_LINEAR) {
        double q = pad_coordinate_d(p, n, padding, align_corners);
        double fl = floor(q);
        double frac = q - fl; /* exact */
        int64_t i0 = (int64_t)fl;
        t->count = 2;
        t->index[0] = i0;
        t->index[1] = i0 + 1;
        t->weight[0] = 1.0 - frac;
        t->weight[1] = frac;
        for (int j = 0; j < 2; ++j)
            t->valid[j] = (t->index[j] >= 0 && t->index[j] < n);
        return 1;
    }

    double fl = floor(p);
    double frac = p - fl;
    int64_t i0 = (int64_t)fl;
    t->count = 4;
    t->weight[0] = keys_kernel(frac + 1.0, OR_CUBIC_A);
    t->weight[1] = keys_kernel(frac, OR_CUBIC_A);
    t->weight[2] = keys_kernel(1.0 - frac, OR_CUBIC_A);
    t->weight[3] = keys_kernel(2.0 - frac, OR_CUBIC_A);
    for (int j = 0; j < 4; ++j) {
        int64_t i = i0 - 1 + j;
        if (padding == OR_PAD_ZEROS) {
            t->index[j] = i;
            t->valid[j] = (i >= 0 && i < n);
        } else if (padding == OR_PAD_BORDER) {
            t->index[j] = i < 0 ? 0 : (i > n - 1 ? n - 1 : i);
            t->valid[j] = 1;
        } else {
            double lo, hi;
            reflect_bounds_d(n, align_corners, &lo, &hi);
            double q = clamp_d(reflect_d((double)i, lo, hi), 0.0, (double)(n - 1));
            t->index[j] = (int64_t)q;
            t->valid[j] = 1;
        }
    }
    return 1;
}

typedef struct {
    const float *X;   /* fp32 X, or */
    const double *Xd; /* float64 X (exactly one of the two is set) */
    int r;
    int64_t N, C;
    const int64_t *in_sp;
    const float *grid;   /* fp32 grid, or */
    const double *gridd; /* float64 grid */
    const int64_t *out_sp;
    int mode, padding, align_corners;
    int64_t in_count, out_count;
} sample_problem;

/* Build the per-axis taps of location (n, o).  Returns 0 when the location
 * contributes nothing (non-finite coordinate). */
static int location_taps(const sample_problem *P, int64_t n, int64_t o, axis_taps *taps)
{
    for (int a = 0; a < P->r; ++a) {
        /* component k of the location vector refers to axis r-1-k */
        int64_t at = (n * P->out_count + o) * P->r + (P->r - 1 - a);
        int ok = P->gridd ? make_axis_taps_d(P->gridd[at], P->in_sp[a], P->mode, P->padding,
                                             P->align_corners, &taps[a])
                          : make_axis_taps(P->grid[at], P->in_sp[a], P->mode, P->padding,
                                           P->align_corners, &taps[a]);
        if (!ok)
            return 0;
    }
    return 1;
}

/* Y[n, c, o] = sum over the product of per-axis taps of
 *   prod_a weight_a * (all taps in range ? X[n, c, index...] : 0). */
static double sample_value(const sample_problem *P, const axis_taps *taps, int64_t n, int64_t c)
{
    const int64_t base = (n * P->C + c) * P->in_count;
    int sel[OR_MAX_RANK];
    for (int a = 0; a < P->r; ++a)
        sel[a] = 0;
    double acc = 0.0;
    for (;;) {
        double w = 1.0;
        int valid = 1;
        int64_t off = 0;
        for (int a = 0; a < P->r; ++a) {
            const axis_taps *t = &taps[a];
            w *= t->weight[sel[a]];
            valid = valid && t->valid[sel[a]];
            off = off * P->in_sp[a] + t->index[sel[a]];
        }
        if (valid)
            acc += w * (P->Xd ? P->Xd[base + off] : (double)P->X[base + off]);
        /* advance the odometer, innermost axis fastest */
        int a = P->r - 1;
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

static int setup_problem(sample_problem *P, const float *X, const double *Xd, int r, int64_t N,
                         int64_t C, const int64_t *in_sp, const float *grid, const double *gridd,
                         const int64_t *out_sp, int mode, int padding, int align_corners)
{
    if (r < 1 || r > OR_MAX_RANK || N < 0 || C < 0)
        return -1;
    if (mode < 0 || mode > 2 || padding < 0 || padding > 2 || (align_corners != 0 && align_corners != 1))
        return -1;
    if (!X == !Xd || !grid == !gridd)
        return -1;
    P->X = X;
    P->Xd = Xd;
    P->r = r;
    P->N = N;
    P->C = C;
    P->in_sp = in_sp;
    P->grid = grid;
    P->gridd = gridd;
    P->out_sp = out_sp;
    P->mode = mode;
    P->padding = padding;
    P->align_corners = align_corners;
    P->in_count = 1;
    P->out_count = 1;
    for (int a = 0; a < r; ++a) {
        if (in_sp[a] < 1 || out_sp[a] < 0)
            return -1;
        P->in_count *= in_sp[a];
        P->out_count *= out_sp[a];
    }
    return 0;
}

/*
 * X: (N, C, in_spatial...) fp32.  grid: (N, out_spatial..., r) fp32.
 * Y: (N, C, out_spatial...) float64, every element written.
 * mode: 0 linear, 1 nearest, 2 cubic.  padding: 0 zeros, 1 border,
 * 2 reflection.  Returns 0, or -1 on a bad argument.
 */
int oracle_grid_sample(const float *X, int r, int64_t N, int64_t C, const int64_t *in_spatial,
                       const float *grid, const int64_t *out_spatial, int mode, int padding,
                       int align_corners, double *Y)
{
    return oracle_grid_sample_ex(X, NULL, r, N, C, in_spatial, grid, NULL, out_spatial, mode,
                                 padding, align_corners, Y);
}

/*
 * General form: X given either as fp32 (X) or as float64 (Xd), the grid
 * either as fp32 (grid) or as float64 (gridd); exactly one of each pair is
 * non-NULL.  A float64 grid takes the coordinate steps in float64.
 */
int oracle_grid_sample_ex(const float *X, const double *Xd, int r, int64_t N, int64_t C,
                          const int64_t *in_spatial, const float *grid, const double *gridd,
                          const int64_t *out_spatial, int mode, int padding, int align_corners,
                          double *Y)
{
    sample_problem P;
    if (setup_problem(&P, X, Xd, r, N, C, in_spatial, grid, gridd, out_spatial, mode, padding,
                      align_corners))
        return -1;
    OR_PARALLEL_FOR
    for (int64_t no = 0; no < N * P.out_count; ++no) {
        const int64_t n = no / P.out_count, o = no % P.out_count;
        axis_taps taps[OR_MAX_RANK];
        int live = location_taps(&P, n, o, taps);
        for (int64_t c = 0; c < C; ++c) {
            double v = live ? sample_value(&P, taps, n, c) : 0.0;
            Y[(n * C + c) * P.out_count + o] = v;
        }
    }
    return 0;
}

/*
 * Same as oracle_grid_sample, but only for the `count` output elements whose
 * flat indices into Y (N, C, out_spatial...) are listed in `flat`; the values
 * go to Y[0..count).  Returns 0, or -1 on a bad argument or index.
 */
int oracle_grid_sample_points(const float *X, int r, int64_t N, int64_t C,
                              const int64_t *in_spatial, const float *grid,
                              const int64_t *out_spatial, int mode, int padding, int align_corners,
                              const int64_t *flat, int64_t count, double *Y)
{
    return oracle_grid_sample_points_ex(X, NULL, r, N, C, in_spatial, grid, NULL, out_spatial,
                                        mode, padding, align_corners, flat, count, Y);
}

/* General form of oracle_grid_sample_points (see oracle_grid_sample_ex). */
int oracle_grid_sample_points_ex(const float *X, const double *Xd, int r, int64_t N, int64_t C,
                                 const int64_t *in_spatial, const float *grid,
                                 const double *gridd, const int64_t *out_spatial, int mode,
                                 int padding, int align_corners, const int64_t *flat,
                                 int64_t count, double *Y)
{
    sample_problem P;
    if (setup_problem(&P, X, Xd, r, N, C, in_spatial, grid, gridd, out_spatial, mode, padding,
                      align_corners))
        return -1;
    for (int64_t i = 0; i < count; ++i)
        if (flat[i] < 0 || flat[i] >= N * C * P.out_count)
            return -1;
    OR_PARALLEL_FOR
    for (int64_t i = 0; i < count; ++i) {
        axis_taps taps[OR_MAX_RANK];
        int64_t f = flat[i];
        int64_t o = f % P.out_count;
        int64_t nc = f / P.out_count;
        int64_t c = nc % C;
        int64_t n = nc / C;
        Y[i] = location_taps(&P, n, o, taps) ? sample_value(&P, taps, n, c) : 0.0;
    }
    return 0;
}
