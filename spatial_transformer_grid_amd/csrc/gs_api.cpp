// gs_api.cpp -- C ABI of libgsample: argument validation and kernel dispatch.
//
// Every check runs before any launch; a rejected call leaves all memory
// untouched.  The library holds no state and allocates nothing: scratch
// memory (DeformConv's channels-last copies) comes from the caller.
#include "gsample.h"
#include "gs_launch.hpp"

#include <math.h>
#include <stdint.h>

namespace {

constexpr int64_t kPlaneLimit = int64_t(1) << 28;   // elements per input/output plane
constexpr int64_t kMaxBlocks = int64_t(1) << 24;    // thread blocks per launch
constexpr int64_t kInt32Max = 0x7fffffff;
constexpr int kBlockThreads = 256;
constexpr int64_t kTargetBlocks = 2048;      // any-rank kernel and Resize
constexpr int64_t kTargetBlocks2D = 4096;    // the 2D sampler
constexpr int64_t kTargetBlocks3D = 1024;    // the 3D sampler

int elem_bytes(int dtype) {
    switch (dtype) {
    case GS_F16: case GS_BF16: case GS_I16: case GS_U16: return 2;
    case GS_F64: case GS_I64: case GS_U64: return 8;
    case GS_I8: case GS_U8: return 1;
    default: return 4;
    }
}

// element types of the tuned sampler and of Resize
bool valid_x_dtype(int d) { return d == GS_F32 || d == GS_F16 || d == GS_BF16; }
// every numeric type GridSample accepts for X
bool valid_any_dtype(int d) { return d >= GS_F32 && d <= GS_U64; }
bool valid_grid_dtype(int d) { return d == GS_F32 || d == GS_F16 || d == GS_BF16 || d == GS_F64; }

int check_attrs(int mode, int padding, int align_corners) {
    if (mode < GS_MODE_LINEAR || mode > GS_MODE_CUBIC) return GS_ERR_ATTR;
    if (padding < GS_PAD_ZEROS || padding > GS_PAD_REFLECTION) return GS_ERR_ATTR;
    if (align_corners != 0 && align_corners != 1) return GS_ERR_ATTR;
    return GS_OK;
}

// product of `n` non-negative extents; false if it exceeds `limit`
bool product_within(const int64_t *e, int n, int64_t limit, int64_t *out) {
    int64_t p = 1;
    for (int i = 0; i < n; ++i) {
        if (e[i] < 0) return false;
        if (e[i] != 0 && p > limit / e[i]) return false;
        p *= e[i];
    }
    *out = p;
    return true;
}

struct Extents {
    int d, h, w;
};

Extents spatial3(const int64_t *sp, int r) {
    Extents e;
    e.d = r == 3 ? (int)sp[0] : 1;
    e.h = (int)sp[r - 2];
    e.w = (int)sp[r - 1];
    return e;
}

int hip_status(int rc) { return rc == 0 ? GS_OK : GS_ERR_HIP; }

// Workspace of the 2D gather path: an 8,448-byte header (kProbes verdict
// words, then the gather kernel's 64 tile counters on separate 128-byte
// lines), then X in channels-last slices
// of 64 (or 32) bytes of channels.  0
// when the path does not apply: it needs fp32 / fp16 / bf16 X whose channels
// fill whole 32-byte slices, an image of X and the channel planes of an image
// of Y each below 2^31 bytes.
constexpr int64_t kGatherHeaderBytes = 8448;  // 64 verdict words, then 64 counters 128 bytes apart

// Launch layout of the gather path: bytes of channels per slice (64 when the
// channels fill them: fewer, longer loads per tap; else 32), (image, slice)
// planes, tiles per plane (output rows x 256-lane row segments) and the tile
// count the gather kernel hands out (planes rounded up to a multiple of the 8
// XCDs when there are at least 8).
struct GatherLayout {
    int slice_bytes;
    int64_t pairs, tiles_per_pair, blocks;
};

// True when the gather path applies to these shapes, with its layout.
bool gather_layout(int x_dtype, const int64_t *x_shape, const int64_t *out_sp, GatherLayout *L) {
    if (!valid_x_dtype(x_dtype)) return false;
    const int bytes = elem_bytes(x_dtype);
    const int64_t N = x_shape[0], C = x_shape[1];
    if (N < 1 || C < 1 || (C * bytes) % 32 != 0) return false;
    int64_t img = 0, outp = 0;
    if (!product_within(x_shape + 1, 3, kInt32Max / bytes, &img) || img == 0) return false;
    const int64_t co[3] = {C, out_sp[0], out_sp[1]};
    if (!product_within(co, 3, kInt32Max / bytes, &outp)) return false;
    if (N > (int64_t(1) << 40) / (img * bytes)) return false;
    L->slice_bytes = (C * bytes) % 64 == 0 ? 64 : 32;
    const int64_t locs = 256 * 16 / L->slice_bytes;
    L->pairs = N * (C * bytes / L->slice_bytes);
    L->tiles_per_pair = out_sp[0] * ((out_sp[1] + locs - 1) / locs);
    L->blocks = (L->pairs >= 8 ? (L->pairs + 7) / 8 * 8 : L->pairs) * L->tiles_per_pair;
    // the tile counters and indices are 32-bit; beyond this the plain
    // sampler runs alone
    return L->blocks <= kMaxBlocks * 8;
}

int64_t gather_workspace_bytes(int x_dtype, const int64_t *x_shape, const int64_t *out_sp) {
    GatherLayout L;
    if (!gather_layout(x_dtype, x_shape, out_sp, &L)) return 0;
    return kGatherHeaderBytes + x_shape[0] * x_shape[1] * x_shape[2] * x_shape[3] *
                                    elem_bytes(x_dtype);
}

// Shared validation and launch of the sampler (fused or not).  With a large
// enough workspace (2D, unfused) the gather path is enqueued too, and the
// device picks one of the two.
int sample(int r, const void *theta, const void *X, int x_dtype, const int64_t *x_shape,
           const void *grid, const int64_t *out_sp, int mode, int padding, int align_corners,
           void *Y, void *stream, void *workspace = nullptr, int64_t workspace_bytes = 0) {
    for (int i = 0; i < r + 2; ++i)
        if (x_shape[i] < 0) return GS_ERR_SHAPE;
    for (int i = 0; i < r; ++i)
        if (out_sp[i] < 0) return GS_ERR_SHAPE;
    const int64_t N = x_shape[0], C = x_shape[1];
    int64_t in_count = 0, out_count = 0;
    if (N > kInt32Max || C > kInt32Max) return GS_ERR_TOO_LARGE;
    if (!product_within(x_shape + 2, r, kPlaneLimit, &in_count)) return GS_ERR_TOO_LARGE;
    if (!product_within(out_sp, r, kPlaneLimit, &out_count)) return GS_ERR_TOO_LARGE;
    if (N == 0 || C == 0 || out_count == 0) return GS_OK;
    if (in_count == 0) return GS_ERR_SHAPE;
    if (!X || !Y || (!grid && !theta)) return GS_ERR_NULL;
    const Extents in = spatial3(x_shape + 2, r), out = spatial3(out_sp, r);
    int tw, th, td;
    gs::tile_shape(r, mode, out.w, &tw, &th, &td);
    const int q = mode == GS_MODE_CUBIC ? 1 : (r == 2 ? 4 : 2);
    const int64_t tiles_w = (out.w + tw - 1) / tw, tiles_h = (out.h + th - 1) / th,
                  tiles_d = (out.d + td - 1) / td;
    const int64_t tiles = tiles_w * tiles_h * tiles_d;
    if (tiles > kMaxBlocks || N * tiles > kMaxBlocks) return GS_ERR_TOO_LARGE;
    // split the channels over several blocks when there are too few tiles:
    // 2-D launches about 4,096 blocks (two rounds of resident blocks on 256
    // CUs, so one block's set-up overlaps another's copies: 5% faster than
    // 2,048 on stn2d_batch and flow2d_half, 8,192 is slower); 3-D tiles stage
    // more rows per channel, and longer channel loops amortise that better
    // (1,024 measured fastest on the volumetric workload)
    const int64_t target = r == 3 ? kTargetBlocks3D : kTargetBlocks2D;
    int64_t groups = (target + N * tiles - 1) / (N * tiles);
    if (groups > C) groups = C;
    if (groups < 1) groups = 1;
    const int64_t cpg = (C + groups - 1) / groups;
    groups = (C + cpg - 1) / cpg;

    const int bytes = elem_bytes(x_dtype);
    const bool vec_in = in.w % gs::stage_chunk_elems(bytes) == 0 && (uintptr_t)X % 16 == 0;
    gs::SampleParams p;
    p.X = X;
    p.Y = Y;
    p.grid = (const float *)grid;
    p.theta = (const float *)theta;
    p.N = (int)N;
    p.C = (int)C;
    p.in_d = in.d;
    p.in_h = in.h;
    p.in_w = in.w;
    p.out_d = out.d;
    p.out_h = out.h;
    p.out_w = out.w;
    p.out_count = (uint32_t)out_count;
    p.in_plane_bytes = (uint32_t)(in_count * bytes);
    p.out_plane_bytes = (uint32_t)(out_count * bytes);
    p.align_corners = align_corners;
    p.tile_w = tw;
    p.tile_h = th;
    p.tile_d = td;
    p.lanes_row_log2 = __builtin_ctz((unsigned)(tw / q));
    p.tile_h_log2 = __builtin_ctz((unsigned)th);
    p.tiles_w = (int)tiles_w;
    p.tiles_h = (int)tiles_h;
    p.tiles_d = (int)tiles_d;
    p.tiles_per_n = (int)tiles;
    p.cgroups = (int)groups;
    p.cpg = (int)cpg;
    p.nblocks = (int)(N * groups * tiles);
    p.vec_out = q > 1 && out.w % q == 0 && (uintptr_t)Y % (uintptr_t)(q * bytes) == 0;
    p.vec_grid = r == 2 && q == 4 && grid != nullptr && out.w % 4 == 0 && (uintptr_t)grid % 16 == 0;
    p.gather_verdicts = nullptr;
    // runs of 16 tiles dealt to the XCDs in turn (one 128 x 128 image of a
    // channel group per run); 32 for images of more tiles, whose footprints
    // then share more of one XCD's L2 (2% faster on 256 x 256 half-precision
    // flows, the same on volumes)
    p.run = tiles > 16 ? 32 : 16;
    if (r == 2 && !theta && workspace && (uintptr_t)workspace % 256 == 0) {
        const int64_t need = gather_workspace_bytes(x_dtype, x_shape, out_sp);
        GatherLayout L;
        if (need > 0 && workspace_bytes >= need && gather_layout(x_dtype, x_shape, out_sp, &L)) {
            gs::GatherParams g;
            g.verdicts = (int *)workspace;
            g.counters = (int *)((char *)workspace + 256);
            g.Xt = (char *)workspace + kGatherHeaderBytes;
            g.slice_bytes = L.slice_bytes;
            g.pairs = (int)L.pairs;
            g.tiles_per_pair = (int)L.tiles_per_pair;
            g.xcd_pairs = L.pairs >= 8;
            g.gather_blocks = (int)L.blocks;
            p.gather_verdicts = g.verdicts;
            // probe, sampler (returns at once when the probe chose the
            // gather path), copy and gather (return at once otherwise)
            const bool vec_x = in.w % (16 / bytes) == 0 && (uintptr_t)X % 16 == 0;
            const hipStream_t st = (hipStream_t)stream;
            int rc = gs::launch_grid_gather(p, g, mode, padding, x_dtype, vec_x, 0, st);
            if (rc) return hip_status(rc);
            rc = gs::launch_grid_sample(p, r, false, mode, padding, x_dtype, vec_in, st);
            if (rc) return hip_status(rc);
            return hip_status(gs::launch_grid_gather(p, g, mode, padding, x_dtype, vec_x, 1, st));
        }
    }
    return hip_status(gs::launch_grid_sample(p, r, theta != nullptr, mode, padding, x_dtype,
                                             vec_in, (hipStream_t)stream));
}

// Validation and launch of the any-rank, any-type sampler.
int sample_nd(int r, const void *X, int x_dtype, const int64_t *x_shape, const void *grid,
              int grid_dtype, const int64_t *out_sp, int mode, int padding, int align_corners,
              void *Y, void *stream) {
    for (int i = 0; i < r + 2; ++i)
        if (x_shape[i] < 0) return GS_ERR_SHAPE;
    const int64_t N = x_shape[0], C = x_shape[1];
    const int bytes = elem_bytes(x_dtype);
    int64_t in_count = 0, out_count = 0;
    if (N > kInt32Max || C > kInt32Max) return GS_ERR_TOO_LARGE;
    if (!product_within(x_shape + 2, r, kPlaneLimit, &in_count)) return GS_ERR_TOO_LARGE;
    if (!product_within(out_sp, r, kPlaneLimit, &out_count)) return GS_ERR_TOO_LARGE;
    if (in_count * bytes > (int64_t(1) << 30) || out_count * bytes > (int64_t(1) << 30))
        return GS_ERR_TOO_LARGE;
    if (N == 0 || C == 0 || out_count == 0) return GS_OK;
    if (in_count == 0) return GS_ERR_SHAPE;
    if (!X || !Y || !grid) return GS_ERR_NULL;
    const int64_t locs = (int64_t)kBlockThreads * gs::nd_locs_per_lane(r, mode);
    const int64_t tiles = (out_count + locs - 1) / locs;
    if (N * tiles > kMaxBlocks) return GS_ERR_TOO_LARGE;
    int64_t groups = (kTargetBlocks + N * tiles - 1) / (N * tiles);
    if (groups > C) groups = C;
    if (groups < 1) groups = 1;
    const int64_t cpg = (C + groups - 1) / groups;
    groups = (C + cpg - 1) / cpg;
    if (N * groups * tiles > kMaxBlocks) return GS_ERR_TOO_LARGE;
    gs::NdParams p;
    p.X = X;
    p.Y = Y;
    p.grid = grid;
    p.x_dtype = x_dtype;
    p.grid_dtype = grid_dtype;
    p.N = (int)N;
    p.C = (int)C;
    for (int a = 0; a < 6; ++a) p.in_ext[a] = a < r ? (int)x_shape[2 + a] : 1;
    p.out_count = (uint32_t)out_count;
    p.in_plane_bytes = (uint32_t)(in_count * bytes);
    p.out_plane_bytes = (uint32_t)(out_count * bytes);
    p.padding = padding;
    p.align_corners = align_corners;
    p.tiles = (int)tiles;
    p.cgroups = (int)groups;
    p.cpg = (int)cpg;
    p.nblocks = (int)(N * groups * tiles);
    return hip_status(gs::launch_grid_sample_nd(p, r, mode, grid_dtype == GS_F64,
                                                (hipStream_t)stream));
}

// GridSample with r spatial axes: the tuned kernels for fp32 / fp16 / bf16 X
// with an fp32 grid in 2D and 3D, the any-rank kernel otherwise.
int grid_sample_rank(int r, const void *X, int x_dtype, const int64_t *x_shape, const void *grid,
                     int grid_dtype, const int64_t *grid_shape, int mode, int padding,
                     int align_corners, void *Y, void *stream) {
    if (!x_shape || !grid_shape) return GS_ERR_NULL;
    if (!valid_any_dtype(x_dtype) || !valid_grid_dtype(grid_dtype)) return GS_ERR_DTYPE;
    int rc = check_attrs(mode, padding, align_corners);
    if (rc) return rc;
    for (int i = 0; i < r + 2; ++i)
        if (grid_shape[i] < 0) return GS_ERR_SHAPE;
    if (grid_shape[0] != x_shape[0] || grid_shape[r + 1] != r) return GS_ERR_SHAPE;
    if ((r == 2 || r == 3) && valid_x_dtype(x_dtype) && grid_dtype == GS_F32)
        return sample(r, nullptr, X, x_dtype, x_shape, grid, grid_shape + 1, mode, padding,
                      align_corners, Y, stream);
    return sample_nd(r, X, x_dtype, x_shape, grid, grid_dtype, grid_shape + 1, mode, padding,
                     align_corners, Y, stream);
}

// Axis index from a possibly negative `axes` entry; -1 when out of range.
int norm_axis(int64_t a, int rank) {
    if (a < 0) a += rank;
    return a >= 0 && a < rank ? (int)a : -1;
}

}  // namespace

extern "C" {

int gs_abi_version(void) { return GS_ABI_VERSION; }

const char *gs_status_string(int status) {
    switch (status) {
    case GS_OK: return "ok";
    case GS_ERR_NULL: return "a required pointer is NULL";
    case GS_ERR_SHAPE: return "inconsistent or negative shape";
    case GS_ERR_DTYPE: return "unsupported element type";
    case GS_ERR_ATTR: return "mode, padding or align_corners out of range";
    case GS_ERR_LAYOUT: return "tensor layout other than dense row-major (reserved)";
    case GS_ERR_TOO_LARGE: return "tensor too large for the kernels' indexing";
    case GS_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
    }
}

int gs_affine_grid(const void *theta, int theta_dtype, const int64_t *size, int size_len,
                   int align_corners, void *grid, void *stream) {
    if (!size) return GS_ERR_NULL;
    if (size_len != 4 && size_len != 5) return GS_ERR_SHAPE;
    if (!valid_grid_dtype(theta_dtype)) return GS_ERR_DTYPE;
    if (align_corners != 0 && align_corners != 1) return GS_ERR_ATTR;
    for (int i = 0; i < size_len; ++i)
        if (size[i] < 0) return GS_ERR_SHAPE;
    const int r = size_len - 2;
    const int64_t N = size[0];
    int64_t count = 0;
    if (N > kInt32Max) return GS_ERR_TOO_LARGE;
    if (!product_within(size + 2, r, kInt32Max, &count)) return GS_ERR_TOO_LARGE;
    if (N == 0 || count == 0) return GS_OK;
    if (!theta || !grid) return GS_ERR_NULL;
    const int64_t tiles = (count + gs::kAffineLocs - 1) / gs::kAffineLocs;
    if (tiles > kMaxBlocks || N * tiles > kMaxBlocks) return GS_ERR_TOO_LARGE;
    const Extents out = spatial3(size + 2, r);
    gs::AffineParams p;
    p.theta = theta;
    p.grid = grid;
    p.theta_dtype = theta_dtype;
    p.N = (int)N;
    p.out_d = out.d;
    p.out_h = out.h;
    p.out_w = out.w;
    p.out_count = (uint32_t)count;
    p.align_corners = align_corners;
    p.tiles_per_n = (int)tiles;
    p.nblocks = (int)(N * tiles);
    gs::FastDivHost dw = gs::make_fastdiv((uint32_t)out.w), dh = gs::make_fastdiv((uint32_t)out.h);
    p.div_w_m = dw.m;
    p.div_w_s = dw.s;
    p.div_h_m = dh.m;
    p.div_h_s = dh.s;
    return hip_status(gs::launch_affine_grid(p, r, (hipStream_t)stream));
}

int gs_grid_sample_2d(const void *X, int x_dtype, const int64_t *x_shape, const void *grid,
                      int grid_dtype, const int64_t *grid_shape, int mode, int padding,
                      int align_corners, void *Y, void *stream) {
    return grid_sample_rank(2, X, x_dtype, x_shape, grid, grid_dtype, grid_shape, mode, padding,
                            align_corners, Y, stream);
}

int gs_grid_sample_2d_workspace_size(int x_dtype, const int64_t *x_shape,
                                     const int64_t *grid_shape, int64_t *bytes) {
    if (!x_shape || !grid_shape || !bytes) return GS_ERR_NULL;
    if (!valid_any_dtype(x_dtype)) return GS_ERR_DTYPE;
    for (int i = 0; i < 4; ++i)
        if (x_shape[i] < 0 || grid_shape[i] < 0) return GS_ERR_SHAPE;
    if (grid_shape[0] != x_shape[0] || grid_shape[3] != 2) return GS_ERR_SHAPE;
    *bytes = gather_workspace_bytes(x_dtype, x_shape, grid_shape + 1);
    return GS_OK;
}

int gs_grid_sample_2d_ws(const void *X, int x_dtype, const int64_t *x_shape, const void *grid,
                         int grid_dtype, const int64_t *grid_shape, int mode, int padding,
                         int align_corners, void *Y, void *workspace, int64_t workspace_bytes,
                         void *stream) {
    if (!x_shape || !grid_shape) return GS_ERR_NULL;
    if (workspace_bytes < 0) return GS_ERR_ATTR;
    if (!valid_x_dtype(x_dtype) || grid_dtype != GS_F32)
        return grid_sample_rank(2, X, x_dtype, x_shape, grid, grid_dtype, grid_shape, mode,
                                padding, align_corners, Y, stream);
    if (!valid_grid_dtype(grid_dtype)) return GS_ERR_DTYPE;
    int rc = check_attrs(mode, padding, align_corners);
    if (rc) return rc;
    for (int i = 0; i < 4; ++i)
        if (grid_shape[i] < 0) return GS_ERR_SHAPE;
    if (grid_shape[0] != x_shape[0] || grid_shape[3] != 2) return GS_ERR_SHAPE;
    return sample(2, nullptr, X, x_dtype, x_shape, grid, grid_shape + 1, mode, padding,
                  align_corners, Y, stream, workspace, workspace_bytes);
}

int gs_grid_sample_3d(const void *X, int x_dtype, const int64_t *x_shape, const void *grid,
                      int grid_dtype, const int64_t *grid_shape, int mode, int padding,
                      int align_corners, void *Y, void *stream) {
    return grid_sample_rank(3, X, x_dtype, x_shape, grid, grid_dtype, grid_shape, mode, padding,
                            align_corners, Y, stream);
}

int gs_grid_sample(const void *X, int x_dtype, const int64_t *x_shape, int x_rank, const void *grid,
                   int grid_dtype, const int64_t *grid_shape, int mode, int padding,
                   int align_corners, void *Y, void *stream) {
    if (x_rank < 3 || x_rank > 8) return GS_ERR_SHAPE;
    return grid_sample_rank(x_rank - 2, X, x_dtype, x_shape, grid, grid_dtype, grid_shape, mode,
                            padding, align_corners, Y, stream);
}

int gs_affine_grid_sample_fused(const void *theta, int theta_dtype, const void *X, int x_dtype,
                                const int64_t *x_shape, int x_rank, const int64_t *out_spatial,
                                int mode, int padding, int align_corners, void *Y, void *stream) {
    if (!x_shape || !out_spatial) return GS_ERR_NULL;
    if (x_rank != 4 && x_rank != 5) return GS_ERR_SHAPE;
    if (theta_dtype != GS_F32 || !valid_x_dtype(x_dtype)) return GS_ERR_DTYPE;
    int rc = check_attrs(mode, padding, align_corners);
    if (rc) return rc;
    const int r = x_rank - 2;
    // a NULL theta with work to do is reported by sample() as GS_ERR_NULL
    return sample(r, theta, X, x_dtype, x_shape, nullptr, out_spatial, mode, padding,
                  align_corners, Y, stream);
}

int gs_resize_output_shape(const int64_t *x_shape, int rank, const int64_t *axes, int count,
                           const float *scales, const int64_t *sizes, int keep_aspect_ratio_policy,
                           int64_t *y_shape) {
    if (!x_shape || !y_shape) return GS_ERR_NULL;
    if (scales && sizes) return GS_ERR_ATTR;
    if (!scales && !sizes) return GS_ERR_NULL;
    if (rank < 1 || rank > 8 || count < 0 || count > rank || (!axes && count != rank))
        return GS_ERR_SHAPE;
    if (keep_aspect_ratio_policy < GS_ASPECT_STRETCH ||
        keep_aspect_ratio_policy > GS_ASPECT_NOT_SMALLER)
        return GS_ERR_ATTR;
    int dims[8];
    bool seen[8] = {false, false, false, false, false, false, false, false};
    for (int i = 0; i < count; ++i) {
        const int d = axes ? norm_axis(axes[i], rank) : i;
        if (d < 0 || seen[d]) return GS_ERR_SHAPE;
        seen[d] = true;
        dims[i] = d;
    }
    for (int a = 0; a < rank; ++a)
        if (x_shape[a] < 0) return GS_ERR_SHAPE;
    int64_t out[8];
    for (int a = 0; a < rank; ++a) out[a] = x_shape[a];
    if (scales) {
        for (int i = 0; i < count; ++i) {
            if (!(scales[i] > 0.0f) || !isfinite(scales[i])) return GS_ERR_ATTR;
            // Summary: floor(input extent * scale)
            out[dims[i]] = (int64_t)floor((double)x_shape[dims[i]] * (double)scales[i]);
        }
    } else if (keep_aspect_ratio_policy == GS_ASPECT_STRETCH) {
        for (int i = 0; i < count; ++i) {
            if (sizes[i] < 0) return GS_ERR_SHAPE;
            out[dims[i]] = sizes[i];
        }
    } else {
        // one scale for every listed axis: the smallest (not_larger) or the
        // largest (not_smaller) size / extent ratio
        double s = 0.0;
        for (int i = 0; i < count; ++i) {
            if (sizes[i] < 0 || x_shape[dims[i]] == 0) return GS_ERR_SHAPE;
            const double r = (double)sizes[i] / (double)x_shape[dims[i]];
            const bool take = keep_aspect_ratio_policy == GS_ASPECT_NOT_LARGER ? r < s : r > s;
            if (i == 0 || take) s = r;
        }
        for (int i = 0; i < count; ++i)
            out[dims[i]] = (int64_t)floor(s * (double)x_shape[dims[i]] + 0.5);  // halfway up
    }
    for (int a = 0; a < rank; ++a) y_shape[a] = out[a];
    return GS_OK;
}

int gs_resize(const void *X, int x_dtype, const int64_t *x_shape, int rank, const int64_t *y_shape,
              const float *scales, int mode, int coordinate_transformation_mode, int nearest_mode,
              float cubic_coeff_a, int exclude_outside, void *Y, void *stream) {
    if (!x_shape || !y_shape) return GS_ERR_NULL;
    if (rank < 1 || rank > 8) return GS_ERR_SHAPE;
    if (!valid_x_dtype(x_dtype)) return GS_ERR_DTYPE;
    if (mode < GS_RESIZE_NEAREST || mode > GS_RESIZE_CUBIC) return GS_ERR_ATTR;
    if (coordinate_transformation_mode < GS_CT_HALF_PIXEL ||
        coordinate_transformation_mode > GS_CT_ASYMMETRIC)
        return GS_ERR_ATTR;
    if (nearest_mode < GS_NEAREST_ROUND_PREFER_FLOOR || nearest_mode > GS_NEAREST_CEIL)
        return GS_ERR_ATTR;
    if ((exclude_outside != 0 && exclude_outside != 1) || !isfinite(cubic_coeff_a))
        return GS_ERR_ATTR;
    for (int a = 0; a < rank; ++a) {
        if (x_shape[a] < 0 || y_shape[a] < 0) return GS_ERR_SHAPE;
        if (scales && (!(scales[a] > 0.0f) || !isfinite(scales[a]))) return GS_ERR_ATTR;
    }
    // the resized axes: from the outermost axis that changes to the last
    int first = rank - 1;
    for (int a = 0; a < rank; ++a)
        if (y_shape[a] != x_shape[a] || (scales && scales[a] != 1.0f)) {
            first = a;
            break;
        }
    if (first < rank - 3) return GS_ERR_SHAPE;
    const int s = rank - first;  // 1, 2 or 3 spatial axes
    int64_t planes = 0, in_count = 0, out_count = 0;
    if (!product_within(x_shape, first, kInt32Max, &planes)) return GS_ERR_TOO_LARGE;
    if (!product_within(x_shape + first, s, kPlaneLimit, &in_count)) return GS_ERR_TOO_LARGE;
    if (!product_within(y_shape + first, s, kPlaneLimit, &out_count)) return GS_ERR_TOO_LARGE;
    if (planes == 0 || out_count == 0) return GS_OK;
    if (in_count == 0) return GS_ERR_SHAPE;
    if (!X || !Y) return GS_ERR_NULL;

    gs::ResizeParams p;
    p.X = X;
    p.Y = Y;
    p.P = (int)planes;
    for (int k = 0; k < 3; ++k) {
        // k = 0 is the last axis (W), 1 is H, 2 is D
        gs::ResizeAxis &ax = p.ax[k];
        const int a = rank - 1 - k;
        if (k >= s) {
            ax.n = ax.m = 1;
            ax.scale = ax.lr = 1.0f;
            continue;
        }
        ax.n = (int)x_shape[a];
        ax.m = (int)y_shape[a];
        if (scales) {
            ax.scale = scales[a];
            ax.lr = (float)ax.n * ax.scale;
        } else {
            ax.scale = (float)ax.m / (float)ax.n;
            ax.lr = (float)ax.m;
        }
    }
    p.ct = coordinate_transformation_mode;
    p.nearest_mode = nearest_mode;
    p.exclude_outside = exclude_outside;
    p.cubic_a = cubic_coeff_a;
    const int bytes = elem_bytes(x_dtype);
    p.in_plane_bytes = (uint32_t)(in_count * bytes);
    p.out_plane_bytes = (uint32_t)(out_count * bytes);
    const bool d3 = s == 3;
    // the kernel's mode numbering is the enum's
    const int q = gs::resize_outputs_per_lane(d3, mode);
    int tw, th;
    gs::resize_tile_shape(q, p.ax[0].m, p.ax[1].m, &tw, &th);
    p.tile_w = tw;
    p.tile_h = th;
    p.lanes_row_log2 = __builtin_ctz((unsigned)(tw / q));
    const int64_t tiles_w = (p.ax[0].m + tw - 1) / tw, tiles_h = (p.ax[1].m + th - 1) / th;
    const int64_t tiles = tiles_w * tiles_h * p.ax[2].m;
    if (tiles > kMaxBlocks) return GS_ERR_TOO_LARGE;
    // planes split over enough blocks: upsampling (more outputs than inputs,
    // short input boxes per tile) gains from two rounds of 4,096 blocks,
    // downsampling (four times the input per output) runs best at 2,048
    const int64_t target = out_count > in_count ? kTargetBlocks2D : kTargetBlocks;
    int64_t groups = (target + tiles - 1) / tiles;
    if (groups > planes) groups = planes;
    if (groups < 1) groups = 1;
    const int64_t ppg = (planes + groups - 1) / groups;
    groups = (planes + ppg - 1) / ppg;
    if (groups * tiles > kMaxBlocks) return GS_ERR_TOO_LARGE;
    p.tiles_w = (int)tiles_w;
    p.tiles_h = (int)tiles_h;
    p.tiles_per_plane = (int)tiles;
    p.pgroups = (int)groups;
    p.ppg = (int)ppg;
    p.nblocks = (int)(groups * tiles);
    p.vec_out = q > 1 && p.ax[0].m % q == 0 && (uintptr_t)Y % (uintptr_t)(q * bytes) == 0;
    const bool vec_in = p.ax[0].n % gs::stage_chunk_elems(bytes) == 0 && (uintptr_t)X % 16 == 0;
    return hip_status(gs::launch_resize(p, d3, mode, x_dtype, vec_in, (hipStream_t)stream));
}

namespace {

// Bytes of the channels-last workspace (a copy of X as (N, H, W, C), then W
// packed for the matrix cores); 0 when that kernel does not apply: it needs
// 2-D fp32 / fp16 / bf16 data and conv and offset groups of a multiple of 8
// channels.
constexpr int64_t kWsAlign = 256;
int64_t round_ws(int64_t b) { return (b + kWsAlign - 1) / kWsAlign * kWsAlign; }

bool cl_applies(int r, int dtype, int64_t Cg, int64_t Cog) {
    return r == 2 && dtype != GS_F64 && Cg % 8 == 0 && Cog % 8 == 0;
}

// Channels per chunk of the channels-last kernel: 64 for fp16 / bf16 with
// more than 128 output channels per group (its 8-wave blocks), else 32.
int64_t cl_chunk(int dtype, int64_t OCg) {
    return (dtype == GS_F16 || dtype == GS_BF16) && OCg > 128 ? 64 : 32;
}

// W packed per conv group: output channels rounded up to 32, channels to the
// chunk size
int64_t cl_w2_elems(int64_t group, int64_t OCg, int64_t Cg, int64_t K, int64_t tk) {
    return group * ((OCg + 31) / 32 * 32) * K * ((Cg + tk - 1) / tk * tk);
}

// Shared validation of gs_deform_conv and gs_deform_conv_workspace_size:
// fills p (pointers aside), the rank, and the output count.
int deform_setup(int dtype, const int64_t *x_shape, int x_rank, const int64_t *w_shape,
                 const int64_t *strides, const int64_t *pads, const int64_t *dilations, int group,
                 int offset_group, gs::DeformParams &p, int &r_out, int64_t &N_out) {
    if (!x_shape || !w_shape) return GS_ERR_NULL;
    if (x_rank < 3 || x_rank > 5) return GS_ERR_SHAPE;
    if (dtype != GS_F32 && dtype != GS_F16 && dtype != GS_BF16 && dtype != GS_F64)
        return GS_ERR_DTYPE;
    const int r = x_rank - 2;
    for (int i = 0; i < x_rank; ++i)
        if (x_shape[i] < 0 || w_shape[i] < 0) return GS_ERR_SHAPE;
    const int64_t N = x_shape[0], C = x_shape[1], OC = w_shape[0];
    if (group < 1 || offset_group < 1) return GS_ERR_ATTR;
    if (C < 1 || OC < 1 || C % group || OC % group || C % offset_group ||
        w_shape[1] != C / group)
        return GS_ERR_SHAPE;
    int64_t st[3], pb[3], pe[3], dl[3], ext[3], ks[3], out[3];
    int64_t npos = 1, plane = 1, K = 1;
    for (int a = 0; a < r; ++a) {
        st[a] = strides ? strides[a] : 1;
        dl[a] = dilations ? dilations[a] : 1;
        pb[a] = pads ? pads[a] : 0;
        pe[a] = pads ? pads[r + a] : 0;
        if (st[a] < 1 || dl[a] < 1 || pb[a] < 0 || pe[a] < 0) return GS_ERR_ATTR;
        ext[a] = x_shape[2 + a];
        ks[a] = w_shape[2 + a];
        if (ext[a] < 1 || ks[a] < 1) return GS_ERR_SHAPE;
        // the sampling arithmetic clamps locations beyond 2^24
        if (ext[a] >= (int64_t(1) << 24) || ks[a] * dl[a] >= (int64_t(1) << 24) ||
            pb[a] >= (int64_t(1) << 24) || pe[a] >= (int64_t(1) << 24) || st[a] >= (int64_t(1) << 24))
            return GS_ERR_TOO_LARGE;
        const int64_t span = dl[a] * (ks[a] - 1) + 1;
        const int64_t room = ext[a] + pb[a] + pe[a] - span;
        if (room < 0) return GS_ERR_SHAPE;
        out[a] = room / st[a] + 1;
        npos *= out[a];
        plane *= ext[a];
        K *= ks[a];
    }
    const int bytes = elem_bytes(dtype);
    const int64_t Cg = C / group, OCg = OC / group;
    if (C * plane * bytes > kInt32Max || OC * npos * bytes > kInt32Max ||
        OC * Cg * K * bytes > kInt32Max || N > kInt32Max)
        return GS_ERR_TOO_LARGE;
    p = gs::DeformParams{};
    p.N = (int)N;
    p.C = (int)C;
    p.OC = (int)OC;
    for (int a = 0; a < 3; ++a) {
        p.in_ext[a] = a < r ? (int)ext[a] : 1;
        p.out_ext[a] = a < r ? (int)out[a] : 1;
        p.k_ext[a] = a < r ? (int)ks[a] : 1;
        p.stride[a] = a < r ? (int)st[a] : 1;
        p.pad[a] = a < r ? (int)pb[a] : 0;
        p.dil[a] = a < r ? (int)dl[a] : 1;
    }
    p.H = p.in_ext[0];
    p.W = r >= 2 ? p.in_ext[1] : 1;
    p.KH = p.k_ext[0];
    p.KW = r >= 2 ? p.k_ext[1] : 1;
    p.OH = p.out_ext[0];
    p.OW = r >= 2 ? p.out_ext[1] : 1;
    p.sh = p.stride[0];
    p.sw = p.stride[1];
    p.pt = p.pad[0];
    p.pl = p.pad[1];
    p.dh = p.dil[0];
    p.dw = p.dil[1];
    p.group = group;
    p.og = offset_group;
    p.Cg = (int)Cg;
    p.OCg = (int)OCg;
    p.Cog = (int)(C / offset_group);
    p.Ktot = (int)(Cg * K);
    int span = 1;
    for (int64_t G = 0; G < group; ++G) {
        const int64_t first = (G * Cg) / p.Cog, last = ((G + 1) * Cg - 1) / p.Cog;
        if (last - first + 1 > span) span = (int)(last - first + 1);
    }
    p.og_span = span;
    p.x_plane_bytes = (uint32_t)(plane * bytes);
    p.w_bytes = (uint32_t)(OC * Cg * K * bytes);
    p.npos = (uint32_t)npos;
    const int64_t tk = cl_chunk(dtype, OCg);
    p.Cgp = (int)((Cg + tk - 1) / tk * tk);
    p.K2 = (int)(K * p.Cgp);
    p.x_img_bytes = (uint32_t)(C * plane * bytes);
    p.Rg = (int)((OCg + 31) / 32);
    const int64_t w2 = cl_w2_elems(group, OCg, Cg, K, tk) * bytes;
    p.w2_bytes = w2 <= kInt32Max ? (uint32_t)w2 : 0;
    p.w2_group_bytes = (uint32_t)(w2 / group);
    // (divisors of at least 1: K, Cgp / tk and C / offset_group are positive here)
    const gs::FastDivHost kkd = gs::make_fastdiv((uint32_t)(K > 0 ? K : 1));
    const gs::FastDivHost cptd = gs::make_fastdiv((uint32_t)(p.Cgp / tk > 0 ? p.Cgp / tk : 1));
    const gs::FastDivHost cogd = gs::make_fastdiv((uint32_t)(p.Cog > 0 ? p.Cog : 1));
    p.kk_m = kkd.m, p.kk_s = kkd.s;
    p.cpt_m = cptd.m, p.cpt_s = cptd.s;
    p.cog_m = cogd.m, p.cog_s = cogd.s;
    r_out = r;
    N_out = N;
    return GS_OK;
}

int64_t cl_workspace_bytes(const gs::DeformParams &p, int r, int dtype) {
    if (!cl_applies(r, dtype, p.Cg, p.Cog) || p.w2_bytes == 0) return 0;
    return round_ws((int64_t)p.N * p.x_img_bytes) + round_ws(p.w2_bytes);
}

}  // namespace

int gs_deform_conv_workspace_size(int dtype, const int64_t *x_shape, int x_rank,
                                  const int64_t *w_shape, const int64_t *strides,
                                  const int64_t *pads, const int64_t *dilations, int group,
                                  int offset_group, int64_t *bytes) {
    if (!bytes) return GS_ERR_NULL;
    gs::DeformParams p;
    int r;
    int64_t N;
    const int rc = deform_setup(dtype, x_shape, x_rank, w_shape, strides, pads, dilations, group,
                                offset_group, p, r, N);
    if (rc != GS_OK) return rc;
    *bytes = cl_workspace_bytes(p, r, dtype);
    return GS_OK;
}

int gs_deform_conv(const void *X, int dtype, const int64_t *x_shape, int x_rank, const void *W,
                   const int64_t *w_shape, const void *offset, const void *B, const void *mask,
                   const int64_t *strides, const int64_t *pads, const int64_t *dilations,
                   int group, int offset_group, void *Y, void *workspace, int64_t workspace_bytes,
                   void *stream) {
    gs::DeformParams p;
    int r;
    int64_t N;
    const int rc = deform_setup(dtype, x_shape, x_rank, w_shape, strides, pads, dilations, group,
                                offset_group, p, r, N);
    if (rc != GS_OK) return rc;
    if (workspace_bytes < 0) return GS_ERR_ATTR;
    if (N == 0) return GS_OK;
    if (!X || !W || !offset || !Y) return GS_ERR_NULL;
    p.X = X;
    p.Wt = W;
    p.offset = offset;
    p.mask = mask;
    p.B = B;
    p.Y = Y;
    p.w_vec = (p.Ktot * elem_bytes(dtype)) % 16 == 0 && (uintptr_t)W % 16 == 0;
    const int64_t need = cl_workspace_bytes(p, r, dtype);
    int path = gs::DC_PATH_DIRECT;
    if (need > 0 && workspace && workspace_bytes >= need && (uintptr_t)workspace % kWsAlign == 0) {
        path = gs::DC_PATH_CL;
        p.Xt = workspace;
        p.W2 = (char *)workspace + round_ws((int64_t)p.N * p.x_img_bytes);
    } else if (r == 2 && dtype != GS_F64) {
        path = gs::DC_PATH_GATHER;
    }
    if (path != gs::DC_PATH_DIRECT) {
        const int64_t tm = p.OCg > 128 ? 256 : 128;
        const int64_t m_tiles = (p.OCg + tm - 1) / tm, n_tiles = ((int64_t)p.npos + 63) / 64;
        const int64_t nblocks = N * group * m_tiles * n_tiles;
        if (nblocks > kMaxBlocks) return GS_ERR_TOO_LARGE;
        p.m_tiles = (int)m_tiles;
        p.n_tiles = (int)n_tiles;
        p.nblocks = (int)nblocks;
    } else {
        const int64_t total = N * p.OC * (int64_t)p.npos;
        if ((total + kBlockThreads - 1) / kBlockThreads > kInt32Max) return GS_ERR_TOO_LARGE;
        p.m_tiles = p.n_tiles = p.nblocks = 0;
    }
    return hip_status(gs::launch_deform_conv(p, r, dtype, path, (hipStream_t)stream));
}

}  // extern "C"
