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
 * writes the grid: gs_affine_grid_sample_fused; and the axis-aligned special
 * case of the sampler, the "Resize" operator (version 18): gs_resize and
 * gs_resize_output_shape; and DeformConv (version 22), whose offset-tap
 * sampling is the same zero-padded linear gather feeding a convolution:
 * gs_deform_conv.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers are DEVICE pointers to dense, contiguous, row-major
 *   tensors owned by the caller.  Shape arrays are HOST memory, read only
 *   during the call.
 * - A tensor pointer needs only the alignment of its element type.  The
 *   library takes 8- and 16-byte accesses where a pointer and the row lengths
 *   allow them and element accesses elsewhere, with the same results bit for
 *   bit.  A workspace is used only when it is 256-byte aligned; otherwise the
 *   call runs the path that needs none.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *   The library allocates no memory (scratch space comes from the caller),
 *   keeps no state between calls and never synchronises; a call returns once
 *   its kernels are enqueued.
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

#define GS_ABI_VERSION 2

/* Status codes.  Every entry point returns an int holding one of them (an
 * enum passed as int keeps the ABI independent of the compiler's enum
 * size).  GS_ERR_LAYOUT is reserved for strided tensors and is never
 * returned: every tensor is dense and row-major. */
typedef enum {
    GS_OK = 0,
    GS_ERR_NULL = 1,      /* a required pointer is NULL while its tensor is non-empty */
    GS_ERR_SHAPE = 2,     /* shapes inconsistent with each other or negative */
    GS_ERR_DTYPE = 3,     /* unsupported element type or type combination */
    GS_ERR_ATTR = 4,      /* mode / padding / align_corners out of range */
    GS_ERR_LAYOUT = 5,    /* reserved: a tensor layout other than dense row-major */
    GS_ERR_TOO_LARGE = 6, /* an extent exceeds what the kernels index */
    GS_ERR_HIP = 7        /* the HIP runtime reported an error at launch */
} gs_status;

/* Element types (GridSample page, Type Constraints; bfloat16 from version 22):
 * X / Y of GridSample may be any of them; grids are GS_F32, GS_F16, GS_BF16
 * or GS_F64; Resize takes GS_F32, GS_F16 and GS_BF16; theta of
 * gs_affine_grid is GS_F32, GS_F16, GS_BF16 or GS_F64 (the grid takes its
 * type), theta of gs_affine_grid_sample_fused is GS_F32.  Types and the
 * enums below are passed as int; the stream is a hipStream_t passed as
 * void *, so the header needs no HIP include. */
typedef enum {
    GS_F32 = 0,
    GS_F16 = 1,
    GS_BF16 = 2,
    GS_F64 = 3,
    GS_I8 = 4,
    GS_U8 = 5,
    GS_I16 = 6,
    GS_U16 = 7,
    GS_I32 = 8,
    GS_U32 = 9,
    GS_I64 = 10,
    GS_U64 = 11
} gs_dtype;

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
 *                element type theta_dtype: GS_F32, GS_F16, GS_BF16 or GS_F64
 *                (Type Constraints: theta and grid share one type).  Row k
 *                maps the homogeneous position (x, y[, z], 1) to component k.
 *                Half types compute in fp32 and round the grid once; GS_F64
 *                computes in double.
 *   size, size_len  host, the output size (N, C, H, W) or (N, C, D, H, W);
 *                C is not used.  All entries >= 0.
 *   align_corners   1: -1 and 1 are the centres of the corner pixels;
 *                0: they are the outer edges of the corner pixels.
 *   grid         device, (N, H, W, 2) or (N, D, H, W, 3), element type
 *                theta_dtype, written whole.
 *                Component 0 is x (along W), 1 is y (along H), 2 is z (along D).
 *
 * Errors: GS_ERR_NULL (theta or grid NULL with N*spatial > 0), GS_ERR_SHAPE
 * (size_len not 4 or 5, negative extent), GS_ERR_DTYPE (theta not a float type),
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
 * Element types: see gs_grid_sample below (any gs_dtype for X; GS_F32,
 * GS_F16, GS_BF16 or GS_F64 grids).
 *
 * Errors: GS_ERR_NULL, GS_ERR_SHAPE (batch mismatch, last grid dim not 2,
 * negative extent, zero input extent with non-empty output), GS_ERR_DTYPE,
 * GS_ERR_ATTR, GS_ERR_TOO_LARGE (an input plane H_in*W_in or an output plane
 * H_out*W_out of more than 2^28 elements or 2^30 bytes, or more than 2^24
 * thread blocks), GS_ERR_HIP.
 */
int gs_grid_sample_2d(const void *X, int x_dtype, const int64_t *x_shape, const void *grid,
                      int grid_dtype, const int64_t *grid_shape, int mode, int padding,
                      int align_corners, void *Y, void *stream);

/*
 * GridSample, 2 spatial dimensions, with a workspace for grids whose
 * locations scatter over the input (GridSample page, as gs_grid_sample_2d).
 * Same arguments, results and errors as gs_grid_sample_2d (GS_ERR_ATTR also
 * for a negative workspace_bytes), plus:
 *
 *   workspace, workspace_bytes   device scratch owned by the caller (256-byte
 *                aligned), at least gs_grid_sample_2d_workspace_size() bytes;
 *                overwritten; not to be shared by calls that may run at the
 *                same time.  NULL, too small or not 256-byte aligned:
 *                exactly gs_grid_sample_2d.
 *
 * With the workspace the call first probes 64 of the sampler's output tiles
 * on the device; when most of them read from more of X than fits a tile's
 * LDS slot (e.g. a random flow), X is copied to channels-last slices of 64
 * bytes of channels (32 when C * sizeof(element) is not a multiple of 64),
 * (N, C / CS, H_in, W_in, CS), in the workspace and sampled from there,
 * several channels per load.  Otherwise the call runs as
 * gs_grid_sample_2d.  Both compute the same taps, weights and fp32 sums in
 * the same order (nearest copies the element bit for bit).  Only fp32 / fp16
 * / bf16 X with an fp32 grid and C * sizeof(element) a multiple of 32 bytes
 * use it; other types run as gs_grid_sample_2d.
 */
int gs_grid_sample_2d_ws(const void *X, int x_dtype, const int64_t *x_shape, const void *grid,
                         int grid_dtype, const int64_t *grid_shape, int mode, int padding,
                         int align_corners, void *Y, void *workspace, int64_t workspace_bytes,
                         void *stream);

/*
 * Bytes of workspace gs_grid_sample_2d_ws can use for these shapes (host
 * only; the grid's values are not read): 8448 + N * C * H_in * W_in *
 * sizeof(element) (an 8,448-byte header of probe verdicts and tile
 * counters, then the copy of X), or 0 when the gather path does not apply
 * (element type, channel bytes, an image or its output planes of 2^31 bytes
 * or more, or more than 2^27 (image, slice, row segment) tiles: then
 * gs_grid_sample_2d_ws runs the plain sampler alone).
 * Written to *bytes.  Errors: GS_ERR_NULL, GS_ERR_DTYPE, GS_ERR_SHAPE
 * (negative extent, batch mismatch, last grid dim not 2).
 */
int gs_grid_sample_2d_workspace_size(int x_dtype, const int64_t *x_shape,
                                     const int64_t *grid_shape, int64_t *bytes);

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
 * GridSample of any rank (GridSample page, Summary: X of rank r+2 with shape
 * (N, C, D1, ..., Dr), grid (N, D1_out, ..., Dr_out, r), Y (N, C, D1_out, ...,
 * Dr_out); the location vector lists the innermost axis first) and any
 * numeric element type (Type Constraints).
 *
 *   X, x_dtype   device, any gs_dtype.  Integer X is interpolated in
 *                floating point and cast at the end (Outputs): truncated
 *                toward zero and saturated to the type's range.
 *   x_shape, x_rank   host, x_rank = r + 2 entries, 1 <= r <= 6.
 *   grid, grid_dtype  device, GS_F32, GS_F16, GS_BF16 (coordinates computed
 *                in fp32 from the exactly widened values) or GS_F64
 *                (coordinates in double).
 *   grid_shape   host, x_rank entries; grid_shape[0] == x_shape[0],
 *                grid_shape[x_rank - 1] == r.
 *   mode, padding, align_corners   as for gs_grid_sample_2d.
 *   Y            device, (N, C, grid_shape[1 .. r]), element type x_dtype.
 *
 * fp32 / fp16 / bf16 X with an fp32 grid in 2 or 3 spatial dimensions run
 * the tuned kernels of gs_grid_sample_2d / _3d (fp32 accumulation).  Every
 * other combination runs a direct-gather kernel that sums in double in the
 * order of the definition (weights as products over the axes, outermost
 * first; taps innermost axis fastest).
 *
 * Errors: as gs_grid_sample_2d; GS_ERR_SHAPE also for x_rank outside 3..8.
 */
int gs_grid_sample(const void *X, int x_dtype, const int64_t *x_shape, int x_rank, const void *grid,
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
 *   X, x_dtype   device input, GS_F32, GS_F16 or GS_BF16.
 *   x_shape, x_rank   host, x_rank (4 or 5) entries.
 *   out_spatial  host, (H_out, W_out) or (D_out, H_out, W_out).
 *   Y            device, (N, C, *out_spatial), element type x_dtype.
 *
 * Errors: as gs_affine_grid and gs_grid_sample_2d/_3d.
 */
int gs_affine_grid_sample_fused(const void *theta, int theta_dtype, const void *X, int x_dtype,
                                const int64_t *x_shape, int x_rank, const int64_t *out_spatial,
                                int mode, int padding, int align_corners, void *Y, void *stream);

/* ------------------------------------------------------------------------
 * Resize (Resize page, version 18), without antialias and without
 * tf_crop_and_resize (no region of interest).
 * --------------------------------------------------------------------- */

/* Attributes, mode: nearest (the default), linear (N-linear), cubic (N-cubic). */
typedef enum { GS_RESIZE_NEAREST = 0, GS_RESIZE_LINEAR = 1, GS_RESIZE_CUBIC = 2 } gs_resize_mode;

/* Attributes, coordinate_transformation_mode (half_pixel is the default):
 * the location x_original of output index x along an axis with input extent
 * n, scale s and length_resized L:
 *   half_pixel          (x + 0.5) / s - 0.5
 *   pytorch_half_pixel  L > 1 ? (x + 0.5) / s - 0.5 : 0
 *   align_corners       L > 1 ? x * (n - 1) / (L - 1) : 0
 *   asymmetric          x / s
 * computed in fp32, one rounded operation at a time, left to right. */
typedef enum {
    GS_CT_HALF_PIXEL = 0,
    GS_CT_PYTORCH_HALF_PIXEL = 1,
    GS_CT_ALIGN_CORNERS = 2,
    GS_CT_ASYMMETRIC = 3
} gs_coord_mode;

/* Attributes, nearest_mode (round_prefer_floor is the default): halfway
 * locations go down, halfway locations go up, floor, ceil.  The index is
 * then clamped into [0, n-1]. */
typedef enum {
    GS_NEAREST_ROUND_PREFER_FLOOR = 0,
    GS_NEAREST_ROUND_PREFER_CEIL = 1,
    GS_NEAREST_FLOOR = 2,
    GS_NEAREST_CEIL = 3
} gs_nearest_mode;

/* Attributes, keep_aspect_ratio_policy (stretch is the default). */
typedef enum {
    GS_ASPECT_STRETCH = 0,
    GS_ASPECT_NOT_LARGER = 1,
    GS_ASPECT_NOT_SMALLER = 2
} gs_aspect_policy;

/*
 * Output extents of Resize (Resize page, Summary; Inputs scales / sizes;
 * Attributes axes and keep_aspect_ratio_policy).  Host only, launches nothing.
 *
 *   x_shape, rank  host, the input extents (1 <= rank <= 8).
 *   axes, count    host, the axes that scales / sizes refer to (count
 *                  entries, negative values count from the back, no
 *                  repeats); axes NULL means all axes in order (count ==
 *                  rank).  Other axes keep their extent.
 *   scales         host, count scales (> 0), or NULL.  Extent =
 *                  floor(extent * scale), evaluated in double precision.
 *   sizes          host, count sizes (>= 0), or NULL.  With policy stretch
 *                  the extents are the sizes; not_larger / not_smaller take
 *                  one scale, the min / max over the listed axes of
 *                  size / extent, and give round-half-up(scale * extent).
 *   y_shape        host, rank entries, written on success.
 *
 * Exactly one of scales and sizes is given.  Errors: GS_ERR_NULL (x_shape or
 * y_shape NULL, or neither scales nor sizes), GS_ERR_SHAPE (rank or count out
 * of range, bad or repeated axis, negative extent or size), GS_ERR_ATTR (both
 * scales and sizes, a scale not finite and > 0, policy out of range).
 */
int gs_resize_output_shape(const int64_t *x_shape, int rank, const int64_t *axes, int count,
                           const float *scales, const int64_t *sizes, int keep_aspect_ratio_policy,
                           int64_t *y_shape);

/*
 * Resize (Resize page, Summary: every output element is a weighted average
 * of sampling locations of the input; Attributes as the enums above).
 *
 *   X            device, the input, rank axes with extents x_shape, element
 *                type x_dtype (GS_F32, GS_F16, GS_BF16).
 *   x_shape, rank  host, 1 <= rank <= 8.
 *   y_shape      host, rank entries: the output extents (for instance from
 *                gs_resize_output_shape).  Only the last three axes may be
 *                resized; every other axis must keep its extent (and scale 1).
 *   scales       host, rank per-axis scales (finite, > 0) when the extents
 *                came from scales, or NULL when they came from sizes.  With
 *                scales, axis a uses s = scales[a] and L = x_shape[a] * s
 *                (fp32, unfloored); without, s = y/x extent (fp32) and L = y
 *                extent.
 *   mode, coordinate_transformation_mode, nearest_mode   the enums above.
 *   cubic_coeff_a  the cubic convolution coefficient a (finite; the page's
 *                default is -0.75).
 *   exclude_outside  0: locations beyond the input take the edge element;
 *                1: their weight is 0 and the remaining weights along that
 *                axis are renormalised to sum 1.
 *   Y            device, extents y_shape, element type x_dtype, written whole.
 *
 * Linear and cubic accumulate in fp32 axis by axis (x innermost); nearest
 * copies the selected element bit for bit.  Errors: GS_ERR_NULL, GS_ERR_SHAPE
 * (rank out of range, negative extent, a resized axis before the last three,
 * a zero input extent with a non-empty output), GS_ERR_DTYPE, GS_ERR_ATTR (an
 * enum out of range, exclude_outside not 0/1, cubic_coeff_a or a scale not
 * finite, a scale <= 0), GS_ERR_TOO_LARGE (the product of the leading axes
 * above 2^31-1, an input or output plane of the resized axes above 2^28
 * elements, more than 2^24 thread blocks), GS_ERR_HIP.
 */
int gs_resize(const void *X, int x_dtype, const int64_t *x_shape, int rank, const int64_t *y_shape,
              const float *scales, int mode, int coordinate_transformation_mode, int nearest_mode,
              float cubic_coeff_a, int exclude_outside, void *Y, void *stream);

/* ------------------------------------------------------------------------
 * DeformConv (DeformConv page, since version 22)
 * --------------------------------------------------------------------- */

/*
 * Y = DeformConv(X, W, offset, B, mask): each kernel position samples X at its
 * regular convolution position plus its offset by linear interpolation (X is
 * zero outside the image), times the mask, times the weight, summed over the
 * input channels of the output channel's group and the kernel positions, plus
 * the bias (Inputs X, W, offset, B, mask; Outputs Y).
 *
 *   X, dtype     device, (N, C, D1 .. Dr), r = x_rank - 2 in 1..3; dtype
 *                GS_F32, GS_F16, GS_BF16 or GS_F64.  W, offset, B, mask and Y
 *                share dtype.
 *   W, w_shape   device (oC, C / group, k1 .. kr); host shape, x_rank entries.
 *   offset       device (N, offset_group * k1*..*kr * r, o1 .. or): for kernel
 *                position k (row-major) of offset group g, channel
 *                g*K*r + k*r + a holds the displacement along axis a, outermost
 *                axis first (the page's examples fix this order).
 *   B            device (oC) or NULL (zeros).
 *   mask         device (N, offset_group * k1*..*kr, o1 .. or) or NULL (ones).
 *   strides, pads, dilations   host, r, 2r (begins then ends) and r entries,
 *                or NULL for 1, 0 and 1 (the page lists no attributes; these
 *                are read with their convolution meaning).
 *   group        input channels split into `group` groups, output channel oc
 *                reading group oc / (oC / group).
 *   offset_group input channel c uses offset group c / (C / offset_group).
 *   Y            device (N, oC, o1 .. or), o_a = (D_a + pad_begin + pad_end -
 *                (dilation * (k_a - 1) + 1)) / stride + 1.
 *
 *   workspace, workspace_bytes   device scratch owned by the caller, or NULL
 *                and 0.  With at least gs_deform_conv_workspace_size() bytes
 *                (256-byte aligned), 2-D fp32 / fp16 / bf16 data whose conv
 *                groups and offset groups hold multiples of 8 channels run on
 *                a channels-last copy of X made there (8 channels per load);
 *                otherwise they gather from X's planes.  Both sum the same
 *                terms in fp32; only the rounding order differs.  The
 *                workspace is overwritten; it must not be shared by calls
 *                that may run at the same time.
 *
 * The sampling location (regular position + offset) is computed in fp32 for
 * fp32 / fp16 / bf16 data and in double for double data.  2-D fp32, fp16 and
 * bf16 run on the matrix cores (MFMA, fp32 accumulation; the sampled values
 * are rounded to the data type before the product); other cases accumulate
 * in double.
 *
 * Errors: GS_ERR_NULL, GS_ERR_SHAPE (x_rank not 3..5, C or oC not divisible
 * by group, C not divisible by offset_group, w_shape[1] != C / group, an
 * empty or too small padded input), GS_ERR_DTYPE, GS_ERR_ATTR (stride or
 * dilation < 1, negative pad, group or offset_group < 1), GS_ERR_TOO_LARGE
 * (an image of X, of Y or all of W above 2^31 - 1 bytes, extents of 2^24 or
 * more, too many thread blocks), GS_ERR_ATTR for a negative workspace_bytes,
 * GS_ERR_HIP.
 */
int gs_deform_conv(const void *X, int dtype, const int64_t *x_shape, int x_rank, const void *W,
                   const int64_t *w_shape, const void *offset, const void *B, const void *mask,
                   const int64_t *strides, const int64_t *pads, const int64_t *dilations,
                   int group, int offset_group, void *Y, void *workspace,
                   int64_t workspace_bytes, void *stream);

/*
 * Bytes of workspace gs_deform_conv uses for these shapes and attributes (the
 * same arguments, same validation and errors), 0 when no workspace helps:
 * N*C*D1*..*Dr elements for X, plus group * (oC/group rounded up to 32) *
 * k1*..*kr * (C/group rounded up to the chunk, 64 for fp16 / bf16 with more
 * than 128 output channels per group, else 32) for W, each part rounded up
 * to 256 bytes.  Written to *bytes (host).
 */
int gs_deform_conv_workspace_size(int dtype, const int64_t *x_shape, int x_rank,
                                  const int64_t *w_shape, const int64_t *strides,
                                  const int64_t *pads, const int64_t *dilations, int group,
                                  int offset_group, int64_t *bytes);

/*
 * gs_deform_conv without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments (workspace and
 * workspace_bytes left out), results and errors as gs_deform_conv called with
 * a workspace of gs_deform_conv_workspace_size() bytes.
 *
 * The channels-last kernel's scratch space (the copy of X and the packed W)
 * lives in a 64 MiB device array inside the library: each GPU the library
 * runs on holds its own copy from the first call on that device until the
 * process ends.  Shapes that need more than 64 MiB return GS_ERR_TOO_LARGE
 * (no work is enqueued); shapes that need none (other ranks, types or
 * channel counts) run as gs_deform_conv without a workspace.  The call
 * allocates nothing.  Every call on a GPU shares that GPU's array, which
 * keeps the last call's contents (every call rewrites what it reads): calls
 * that may run at the same time on one GPU (on different streams, or from
 * different threads) race and must be serialised by the caller.
 */
int gs_deform_conv_noalloc(const void *X, int dtype, const int64_t *x_shape, int x_rank,
                           const void *W, const int64_t *w_shape, const void *offset,
                           const void *B, const void *mask, const int64_t *strides,
                           const int64_t *pads, const int64_t *dilations, int group,
                           int offset_group, void *Y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GSAMPLE_H */
