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
    int tiles_w, tiles_h, tiles_d;  // output tiles per image along W, H, D
    int tiles_per_n;           // tiles_w * tiles_h * tiles_d
    int cgroups, cpg;          // channel groups per image, channels per group
    int nblocks;               // N * cgroups * tiles_per_n
    int vec_out;               // Y rows allow one vector store per lane
};

// Output tile of one 256-thread block and the number Q of consecutive
// outputs (along W) each lane owns.  2D nearest / linear: 32 x 32 outputs,
// 4 per lane; 2D cubic: 16 x 16, 1 per lane; 3D: 8 x 8 x 4, 1 per lane.
template <int R, int MODE>
struct Geo {
    static constexpr int Q = (R == 2 && MODE != 2) ? 4 : 1;
    static constexpr int w = R == 2 ? (Q == 4 ? 32 : 16) : 8;
    static constexpr int h = R == 2 ? (Q == 4 ? 32 : 16) : 8;
    static constexpr int d = R == 2 ? 1 : 4;
};

// Elements per 16-byte chunk of the LDS staging copy.
inline int stage_chunk_elems(int elem_bytes) { return 16 / elem_bytes; }

struct AffineParams {
    const float *theta;  // (N, R, R+1)
    float *grid;         // (N, out..., R)
    int N;
    int out_d, out_h, out_w;
    uint32_t out_count;
    int align_corners;
    int tiles_per_n;
    int nblocks;
    uint32_t div_w_m, div_w_s;
    uint32_t div_h_m, div_h_s;
};

// Launchers (gs_kernels.hip).  Return 0 on success or the hipError_t of the
// launch.  `rank` is 2 or 3; `dtype` 0 f32, 1 f16, 2 bf16; `vec_in` selects
// 16-byte staging loads (input rows a whole number of 16-byte chunks).
int launch_grid_sample(const SampleParams &p, int rank, bool fused, int mode, int padding,
                       int dtype, bool vec_in, hipStream_t stream);
int launch_affine_grid(const AffineParams &p, int rank, hipStream_t stream);

}  // namespace gs
