/*
 * gsample.h -- C ABI of libgsample, the MI355X (gfx950) spatial-transformer
 * grid generator and sampler.
 *
 * The operations are the ONNX operators defined on the pages
 *   "AffineGrid" (since version 20)            -> gs_affine_grid
 *   "GridSample - version 20" / "GridSample"   -> gs_grid_sample_2d / _3d
 *   (version 22 adds bfloat16)
 * plus their composition as the grid generator and sampler of a spatial
 * transformer (GridSample page, Summary), fused into one pass that never
 * writes the grid: gs_affine_grid_sample_fused.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers are DEVICE pointers to dense, contiguous, row-major
 *   tensors owned by the caller.  Shape arrays are HOST memory, read only
 *   during the call.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *   The library allocates no memory, keeps no state between calls and never
 *   synchronises; a call returns once its kernel is enqueued.
 * - The output must not overlap any input.
 * - Every argument is validated before anything is launched.  On any error
 *   nothing is launched or written and the status says why.  A tensor with a
 *   zero extent returns GS_OK without launching.
 * - Floating-point semantics: coordinates (grid generation, un-normalisation,
 *   padding) are computed in fp32 one rounded operation at a time, in the
 *   order the page formulas are written (no fused multiply-add), so nearest
 *   mode picks the same pixel as any implementation that follows that order.
 *   Interpolation accumulates in fp32; half-precision outputs are rounded to
 *   nearest even once, at the store.
 * - A sampling location that is NaN or infinite yields 0 (the pages do not
 *   cover it).  Every memory access stays inside its tensor for any grid value.
 */
#ifndef GSAMPLE_H
#define GSAMPLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GS_ABI_VERSION 1

typedef enum {
    GS_OK = 0,
    GS_ERR_NULL = 1,      /* a required pointer is NULL while its tensor is non-empty */
    GS_ERR_SHAPE = 2,     /* shapes inconsistent with each other or negative */
    GS_ERR_DTYPE = 3,     /* unsupported element type or type combination */
    GS_ERR_ATTR = 4,      /* mode / padding / align_corners out of range */
    GS_ERR_TOO_LARGE = 5, /* an extent exceeds what the kernels index */
    GS_ERR_HIP = 6        /* the HIP runtime reported an error at launch */
} gs_status;

/* Element types (GridSample page, Type Constraints; bfloat16 from version 22). */
typedef enum { GS_F32 = 0, GS_F16 = 1, GS_BF16 = 2 } gs_dtype;

/* GridSample page, Attributes, mode: linear (the default; bilinear in 2D,
 * trilinear in 3D), nearest (ties to the even index), cubic (bicubic /
 * tricubic with the cubic convolution kernel, coefficient a = -0.75, the
 * cubic_coeff_a default of the Resize page). */
typedef enum { GS_MODE_LINEAR = 0, GS_MODE_NEAREST = 1, GS_MODE_CUBIC = 2 } gs_mode;

/* GridSample page, Attributes, padding_mode: zeros (the default; locations
 * outside the image read 0), border (they read the edge value), reflection
 * (they are mirrored at the borders until inside).  linear and nearest pad the
 * location; cubic pads each of its taps. */
typedef enum { GS_PAD_ZEROS = 0, GS_PAD_BORDER = 1, GS_PAD_REFLECTION = 2 } gs_padding;

/* Version of this ABI (GS_ABI_VERSION of the build). */
int gs_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char *gs_status_string(int status);

/*
 * AffineGrid (AffineGrid page, Summary; Inputs theta and size; Output grid).
 *
 *   theta        device, (N, 2, 3) for size_len 4 or (N, 3, 4) for size_len 5,
 *                element type theta_dtype (GS_F32 only).  Row k maps the
 *                homogeneous position (x, y[, z], 1) to component k.
 *   size, size_len  host, the output size (N, C, H, W) or (N, C, D, H, W);
 *                C is not used.  All entries >= 0.
 *   align_corners   1: -1 and 1 are the centres of the corner pixels;
 *                0: they are the outer edges of the corner pixels.
 *   grid         device, (N, H, W, 2) or (N, D, H, W, 3) fp32, written whole.
 *                Component 0 is x (along W), 1 is y (along H), 2 is z (along D).
 *
 * Errors: GS_ERR_NULL (theta or grid NULL with N*spatial > 0), GS_ERR_SHAPE
 * (size_len not 4 or 5, negative extent), GS_ERR_DTYPE (theta not GS_F32),
 * GS_ERR_ATTR (align_corners not 0/1), GS_ERR_TOO_LARGE (H*W or D*H*W above
 * 2^31-1, or more than 2^24 thread blocks), GS_ERR_HIP.
 */
int gs_affine_grid(const void *theta, int theta_dtype, const int64_t *size, int size_len,
                   int align_corners, void *grid, void *stream);

/*
 * GridSample, 2 spatial dimensions (GridSample page, Summary, Inputs X and
 * grid, Output Y, Attributes).
 *
 *   X            device, (N, C, H_in, W_in), element type x_dtype.
 *   x_shape      host, 4 entries.
 *   grid         device, (N, H_out, W_out, 2) fp32 (grid_dtype GS_F32);
 *                component 0 is the normalised x (along W), 1 is y (along H).
 *   grid_shape   host, 4 entries; grid_shape[0] == x_shape[0], [3] == 2.
 *   mode, padding, align_corners   as the enums above; align_corners 0/1.
 *   Y            device, (N, C, H_out, W_out), same element type as X,
 *                written whole.
 *
 * Errors: GS_ERR_NULL, GS_ERR_SHAPE (batch mismatch, last grid dim not 2,
 * negative extent, zero input extent with non-empty output), GS_ERR_DTYPE
 * (x_dtype not GS_F32/GS_F16/GS_BF16, grid_dtype not GS_F32), GS_ERR_ATTR,
 * GS_ERR_TOO_LARGE (an input plane H_in*W_in or an output plane H_out*W_out
 * of more than 2^28 elements, or more than 2^24 thread blocks), GS_ERR_HIP.
 */
int gs_grid_sample_2d(const void *X, int x_dtype, const int64_t *x_shape, const void *grid,
                      int grid_dtype, const int64_t *grid_shape, int mode, int padding,
                      int align_corners, void *Y, void *stream);

/*
 * GridSample, 3 spatial dimensions.  As gs_grid_sample_2d with
 *   X (N, C, D_in, H_in, W_in), grid (N, D_out, H_out, W_out, 3) whose
 *   components are x (W), y (H), z (D), Y (N, C, D_out, H_out, W_out);
 *   x_shape and grid_shape hold 5 entries.
 */
int gs_grid_sample_3d(const void *X, int x_dtype, const int64_t *x_shape, const void *grid,
                      int grid_dtype, const int64_t *grid_shape, int mode, int padding,
                      int align_corners, void *Y, void *stream);

/*
 * AffineGrid followed by GridSample in one pass (the grid generator and
 * sampler of a spatial transformer).  Each output location computes its grid
 * vector from theta in registers exactly as gs_affine_grid does (same bits)
 * and samples X with it; the grid is never written to memory.  The result is
 * bit-identical to gs_affine_grid followed by gs_grid_sample_2d/_3d with the
 * same align_corners.
 *
 *   theta        device, (N, 2, 3) (x_rank 4) or (N, 3, 4) (x_rank 5), GS_F32.
 *   X, x_dtype   device input as for gs_grid_sample_2d/_3d.
 *   x_shape, x_rank   host, x_rank (4 or 5) entries.
 *   out_spatial  host, (H_out, W_out) or (D_out, H_out, W_out).
 *   Y            device, (N, C, *out_spatial), element type x_dtype.
 *
 * Errors: as gs_affine_grid and gs_grid_sample_2d/_3d.
 */
int gs_affine_grid_sample_fused(const void *theta, int theta_dtype, const void *X, int x_dtype,
                                const int64_t *x_shape, int x_rank, const int64_t *out_spatial,
                                int mode, int padding, int align_corners, void *Y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GSAMPLE_H */
