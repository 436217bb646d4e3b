// gs_launch.hpp -- parameters passed from the C-ABI layer to the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gs {

struct FastDivHost {
    uint32_t d, m, s;
};

// Multiplier and shift for gs::fdiv (divisors 1 .. 2^31-1, dividends < 2^31).
inline FastDivHost make_fastdiv(uint32_t d) {
    uint32_t s = 0;
    while (s < 32 && (1ull << s) < d) ++s;
    uint64_t m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
    return FastDivHost{d, (uint32_t)m, s};
}

// One sampling launch: 2 or 3 spatial axes, extents listed outermost first;
// for 2D the depth extents are 1.
struct SampleParams {
    const void *X;
    void *Y;
    const float *grid;   // unfused: (N, out..., R)
    const float *theta;  // fused:   (N, R, R+1)
    int N, C;
    int in_d, in_h, in_w;
    int out_d, out_h, out_w;
    uint32_t out_count;        // out_d * out_h * out_w
    uint32_t in_plane_bytes;   // in_d * in_h * in_w * sizeof(T)   (<= 2^30)
    uint32_t out_plane_bytes;  // out_count * sizeof(T)            (<= 2^30)
    int align_corners;
    int tile_w, tile_h, tile_d;     // output tile of one block (powers of two)
    int lanes_row_log2;             // log2(tile_w / Q): lanes per tile row
    int tile_h_log2;                // log2(tile_h)
    int tiles_w, tiles_h, tiles_d;  // output tiles per image along W, H, D
    int tiles_per_n;           // tiles_w * tiles_h * tiles_d
    int cgroups, cpg;          // channel groups per image, channels per group
    int nblocks;               // N * cgroups * tiles_per_n
    int vec_out;               // Y rows allow one vector store per lane
    int vec_grid;              // 2D grid rows allow 16-byte loads of 4 vectors
    const int *gather_verdicts;  // non-NULL: skip when the gather path was chosen
    int run;                   // logical blocks per XCD run (16 or 32)
};

// The 2D gather path on a channels-last copy of X (workspace: kProbes verdict
// words, then Xt in slices of 64 or 32 bytes of channels, (N, C / CS, H, W,
// CS)).
struct GatherParams {
    void *Xt;
    int *verdicts;
    int *counters;             // 64 tile counters of the gather kernel, 128 bytes apart
    int slice_bytes;           // bytes of channels per pixel slice: 64 or 32
    int pairs;                 // N * C / CS (image, slice) planes
    int tiles_per_pair;        // out_h * ceil(out_w / (256 * 16 / slice_bytes))
    int xcd_pairs;             // blocks ordered per XCD (pairs >= 8)
    int gather_blocks;         // launch size
};

// Outputs per lane Q (consecutive along W) and the LDS bytes for staging.
// Nearest / linear: 4 outputs per lane in 2D, 2 in 3D; cubic: 1.
template <int R, int MODE>
struct Geo {
    static constexpr int Q = MODE == 2 ? 1 : (R == 2 ? 4 : 2);
    static constexpr int stage_bytes = 16384;
};

// Output tile of a 256-thread block: 2D nearest / linear 128 x 8 when an
// output row fits in 128 locations (no tile boundary crosses the rows the
// block reads), else 64 x 16, and 32 x 32 for rows of at most 32; 2D cubic
// 16 x 16; 3D nearest / linear 32 x 4 x 4 (each output row segment of a
// block is a whole 128-byte line of fp32 Y); 3D cubic 8 x 8 x 4.  Chosen by
// measurement on the workloads the library is tuned for.
inline void tile_shape(int r, int mode, int out_w, int *w, int *h, int *d) {
    if (r == 2 && mode != 2) {
        *w = out_w > 128 ? 64 : (out_w > 64 ? 128 : (out_w > 32 ? 64 : 32));
        *h = 1024 / *w;
        *d = 1;
    } else if (r == 2) {
        *w = 16, *h = 16, *d = 1;
    } else if (mode != 2) {
        *w = 32, *h = 4, *d = 4;
    } else {
        *w = 8, *h = 8, *d = 4;
    }
}

// Elements per 16-byte chunk of the LDS staging copy.
inline int stage_chunk_elems(int elem_bytes) { return 16 / elem_bytes; }

// Locations per block of the grid generator.
constexpr int kAffineLocs = 1024;

struct AffineParams {
    const void *theta;   // (N, R, R+1), element type theta_dtype
    void *grid;          // (N, out..., R), element type theta_dtype
    int theta_dtype;     // 0 f32, 1 f16, 2 bf16, 3 f64
    int N;
    int out_d, out_h, out_w;
    uint32_t out_count;
    int align_corners;
    int tiles_per_n;
    int nblocks;
    uint32_t div_w_m, div_w_s;
    uint32_t div_h_m, div_h_s;
};

// One resized axis: input and output extent, the scale of the coordinate
// transformation and length_resized (scale * input extent, or the output
// extent when the extents came from sizes).
struct ResizeAxis {
    int n, m;
    float scale, lr;
};

// One Resize launch over P planes of up to 3 resized trailing axes.
struct ResizeParams {
    const void *X;
    void *Y;
    int P;                     // planes: product of the leading (unresized) axes
    ResizeAxis ax[3];          // W, H, D (extent 1 when absent)
    int ct;                    // coordinate_transformation_mode 0..3
    int nearest_mode;          // 0..3
    int exclude_outside;       // 0 / 1
    float cubic_a;
    uint32_t in_plane_bytes, out_plane_bytes;  // each <= 2^30
    int tile_w, tile_h;        // output tile of one block (tile_w / Q lanes per row)
    int lanes_row_log2;
    int tiles_w, tiles_h, tiles_per_plane;     // tiles_per_plane = tiles_w * tiles_h * D_out
    int pgroups, ppg;          // plane groups, planes per group
    int nblocks;               // pgroups * tiles_per_plane
    int vec_out;               // Y rows allow one vector store per lane
};

// Outputs per lane of the Resize kernel (mode 0 nearest, 1 linear, 2 cubic):
// 4 (cubic 2) when at most H and W are resized, 2 (cubic 1) when D is resized
// too.  Cubic holds 16 or 64 taps per output; fewer outputs per lane keep its
// registers, and so its occupancy, in line (measured).
constexpr int resize_outputs_per_lane(bool d3, int mode) {
    return d3 ? (mode == 2 ? 1 : 2) : (mode == 2 ? 2 : 4);
}

// Outputs per lane and LDS staging bytes of the Resize kernel.
template <int MODE, bool D3>
struct RzGeo {
    static constexpr int Q = resize_outputs_per_lane(D3, MODE);
    static constexpr int stage_bytes = 16384;
};

// Resize tile: 16 lanes per row (64 outputs at Q = 4), 32 for rows of 65..128
// outputs, fewer for narrow rows; when the output has few rows the tile is
// widened instead (a 1-D resize uses up to 256 lanes per row).
inline void resize_tile_shape(int q, int out_w, int out_h, int *tw, int *th) {
    int lanes = (q == 4 && out_w > 64 && out_w <= 128) ? 32 : 16;
    while (lanes > 4 && (lanes / 2) * q >= out_w) lanes /= 2;
    int h = 256 / lanes;
    while (h > 1 && h / 2 >= out_h && lanes < 256) {
        h /= 2;
        lanes *= 2;
    }
    *tw = lanes * q;
    *th = h;
}

// Output locations per lane of the any-rank sampler (mode: 0 linear, 1
// nearest, 2 cubic): the per-wave set-up and each channel's buffer ranges
// then serve that many outputs.  Measured on the type workloads: rank-1
// linear 4 (126.6 -> 119.5 us on signal1d_f32; 8 gained 1.5% for twice the
// registers); 2-D linear 2 (182 -> 154 us on stn2d_u8; 4 took 135 VGPRs and
// 227 us); 2-D nearest 4; everything else (3 taps per axis, rank >= 3) 1.
constexpr int nd_locs_per_lane(int rank, int mode) {
    return rank == 1 && mode != 2 ? 4 : (rank == 2 && mode == 1 ? 4 : (rank == 2 && mode == 0 ? 2 : 1));
}

// One launch of the any-rank, any-type sampler (gs_nd.hip).
struct NdParams {
    const void *X;
    void *Y;
    const void *grid;
    int x_dtype;               // 0 f32, 1 f16, 2 bf16, 3 f64, 4 i8, 5 u8, 6 i16, 7 u16,
                               // 8 i32, 9 u32, 10 i64, 11 u64
    int grid_dtype;            // 0 f32, 1 f16, 2 bf16, 3 f64
    int N, C;
    int in_ext[6];             // spatial input extents, outermost first
    uint32_t out_count;        // output locations per image (<= 2^28)
    uint32_t in_plane_bytes, out_plane_bytes;  // each <= 2^30
    int padding, align_corners;
    int tiles;                 // ceil(out_count / (256 * nd_locs_per_lane))
    int cgroups, cpg, nblocks; // channel groups, channels per group, blocks
};

// One DeformConv launch (gs_deform.hip).  2-D uses the H / W / sh ... fields,
// the direct kernel the per-axis arrays (r <= 3 axes, outermost first).
struct DeformParams {
    const void *X, *Wt, *offset, *mask, *B;  // mask and B may be NULL
    void *Y;
    int N, C, OC;
    int H, W, KH, KW, OH, OW;                // 2-D extents
    int sh, sw, pt, pl, dh, dw;              // 2-D strides, pad begins, dilations
    int in_ext[3], out_ext[3], k_ext[3], stride[3], pad[3], dil[3];
    int group, og, Cg, OCg, Cog, Ktot;       // Ktot = Cg * kernel size
    int og_span;                             // offset groups one conv group spans
    int m_tiles, n_tiles, nblocks;
    uint32_t x_plane_bytes;                  // one input plane; C planes < 2^31 bytes
    uint32_t w_bytes;                        // all of W (< 2^31)
    uint32_t npos;                           // output positions per plane
    int w_vec;                               // W rows allow 16-byte loads
    // channels-last path: workspace copies of X (N, H, W, C) and of W packed
    // in the matrix cores' operand order: per conv group Rg = ceil(OCg / 32)
    // blocks of 32 rows x K2 = KH*KW*Cgp, Cgp = Cg rounded up to 32
    void *Xt, *W2;
    int Cgp, K2, Rg;
    uint32_t x_img_bytes;                    // one image of Xt (< 2^31)
    uint32_t w2_group_bytes;                 // one conv group of W2
    uint32_t w2_bytes;                       // all of W2 (< 2^31)
    // multipliers and shifts of gs::fdiv for KK = KH * KW, the chunks per
    // kernel position and Cog (channels-last kernel)
    uint32_t kk_m, kk_s, cpt_m, cpt_s, cog_m, cog_s;
};

// DeformConv kernels: direct (one lane per output, double sums), implicit
// GEMM gathering from X's planes, implicit GEMM on a channels-last copy.
enum { DC_PATH_DIRECT = 0, DC_PATH_GATHER = 1, DC_PATH_CL = 2 };

// Launchers (gs_kernels.hip, gs_resize.hip, gs_nd.hip, gs_deform.hip).  Return 0 on success or the hipError_t of the
// launch.  `rank` is 2 or 3; `dtype` 0 f32, 1 f16, 2 bf16; `vec_in` selects
// 16-byte staging loads (input rows a whole number of 16-byte chunks).
int launch_grid_sample(const SampleParams &p, int rank, bool fused, int mode, int padding,
                       int dtype, bool vec_in, hipStream_t stream);
// The gather path's launches: `part` 0 the probe (before the sampler), 1
// the copy and the gather (after it).
int launch_grid_gather(const SampleParams &p, const GatherParams &g, int mode, int padding,
                       int dtype, bool vec_in, int part, hipStream_t stream);
int launch_affine_grid(const AffineParams &p, int rank, hipStream_t stream);
// `rank` 1..6 spatial axes; `double_grid`: the grid is double (coordinates in
// double), else fp32 / fp16 / bf16 (coordinates in fp32).
int launch_grid_sample_nd(const NdParams &p, int rank, int mode, bool double_grid,
                          hipStream_t stream);
// `mfma`: the 2-D matrix-core kernel (dtype 0 f32, 1 f16, 2 bf16); else the
// direct kernel (rank 1..3, dtype 0..3 with 3 = f64).
int launch_deform_conv(const DeformParams &p, int rank, int dtype, int path, hipStream_t stream);
// `d3`: the third axis from the end is resized; `mode` 0 nearest, 1 linear,
// 2 cubic.
int launch_resize(const ResizeParams &p, bool d3, int mode, int dtype, bool vec_in,
                  hipStream_t stream);

}  // namespace gs
