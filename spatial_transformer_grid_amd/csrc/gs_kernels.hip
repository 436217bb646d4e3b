// gs_kernels.hip -- grid generator and sampler kernels for gfx950.
//
// Layout: one lane owns one output location.  A block of 256 lanes (4 wave64)
// covers 256 consecutive locations of one image in row-major output order, so
// grid reads and Y stores are contiguous across the wavefront.  Each lane
// computes its sampling location, tap offsets and weights once, then walks
// the channels: per channel it gathers its taps from that channel's plane of
// X and stores one value of Y.  Loads of U channels are issued before any of
// their stores, so each lane keeps U * taps loads in flight.
//
// Operator definitions: AffineGrid page (Summary: theta applied to evenly
// spaced positions over [-1, 1]); GridSample page (Summary; Attributes
// align_corners, mode, padding_mode).  Cubic uses the cubic convolution kernel
// with a = -0.75 (the cubic_coeff_a default of the Resize page).
#include "gs_device.hpp"
#include "gs_launch.hpp"

namespace gs {

// Flat output location -> (d, h, w).
template <int R>
__device__ __forceinline__ void decompose(uint32_t l, int out_w, int out_h, uint32_t wm,
                                          uint32_t ws, uint32_t hm, uint32_t hs, int &d, int &h,
                                          int &w) {
    uint32_t row = fdiv(l, FastDiv{0, wm, ws});
    w = (int)(l - row * (uint32_t)out_w);
    if (R == 2) {
        h = (int)row;
        d = 0;
    } else {
        uint32_t dd = fdiv(row, FastDiv{0, hm, hs});
        h = (int)(row - dd * (uint32_t)out_h);
        d = (int)dd;
    }
}

// Grid vector of output location (d, h, w): theta applied to the homogeneous
// base position.  Products and sums are rounded one at a time, summed left
// to right with the translation last; gs_affine_grid and the fused sampler
// both use this function, so they produce the same bits.
template <int R>
__device__ __forceinline__ void affine_vector(const float *th, int d, int h, int w, int out_d,
                                              int out_h, int out_w, int ac, float g[R]) {
    float b[3];
    b[0] = base_position(w, out_w, ac);
    b[1] = base_position(h, out_h, ac);
    b[2] = R == 3 ? base_position(d, out_d, ac) : 0.0f;
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const float *row = th + k * (R + 1);
        float s = row[0] * b[0];
#pragma unroll
        for (int j = 1; j < R; ++j) {
            float prod = row[j] * b[j];
            s = s + prod;
        }
        s = s + row[R];
        g[k] = s;
    }
}

template <int R>
__global__ __launch_bounds__(kBlock) void affine_grid_kernel(AffineParams p) {
    const int lb = xcd_logical_block(p.nblocks);
    if (lb >= p.nblocks) return;
    const int n = lb / p.tiles_per_n;
    const int tile = lb - n * p.tiles_per_n;
    const uint32_t l = (uint32_t)tile * kBlock + threadIdx.x;
    if (l >= p.out_count) return;
    int d, h, w;
    decompose<R>(l, p.out_w, p.out_h, p.div_w_m, p.div_w_s, p.div_h_m, p.div_h_s, d, h, w);
    float g[R];
    affine_vector<R>(p.theta + (size_t)n * R * (R + 1), d, h, w, p.out_d, p.out_h, p.out_w,
                     p.align_corners, g);
    float *out = p.grid + ((size_t)n * p.out_count + l) * R;
#pragma unroll
    for (int k = 0; k < R; ++k) out[k] = g[k];
}

// ------------------------------------------------------------------ taps

// Number of taps per output location and channels per load group.
template <int R, int MODE>
struct Shape {
    static constexpr int taps = MODE == MODE_NEAREST ? 1 : (MODE == MODE_LINEAR ? (1 << R) : 16);
    static constexpr int group = MODE == MODE_NEAREST ? 8
                                 : MODE == MODE_LINEAR ? (R == 2 ? 8 : 4)
                                                       : (R == 2 ? 2 : 1);
};

// Per-location tap offsets (bytes within one plane, GS_OOB when the tap lies
// outside the image or the location is not finite) and weights.
// For 3D cubic the 64 taps are formed per channel from 16 (z, y) row offsets
// and 4 x offsets: off[0..15] = rows, xoff[0..3] = columns.
template <int R, int MODE, int PAD, typename T>
struct Taps {
    uint32_t off[Shape<R, MODE>::taps];
    float w[MODE == MODE_NEAREST ? 1 : Shape<R, MODE>::taps];
    uint32_t xoff[4];
    float wz[4], wyx[4], wx[4];

    __device__ __forceinline__ void build(const float g[R], const int ext[3], int ac) {
        uint32_t stride[3];
        stride[0] = (uint32_t)T::bytes;
        stride[1] = (uint32_t)ext[0] * T::bytes;
        stride[2] = (uint32_t)ext[0] * (uint32_t)ext[1] * T::bytes;
        // pixel coordinates; a non-finite one kills the whole location
        float pc[R];
        bool dead = false;
#pragma unroll
        for (int k = 0; k < R; ++k) {
            float q = unnormalize(g[k], ext[k], ac);
            bool fin = __builtin_isfinite(q);
            dead = dead || !fin;
            pc[k] = fin ? clampf(q, -kCoordLimit, kCoordLimit) : 0.0f;
        }

        if constexpr (MODE == MODE_NEAREST) {
            bool ok = !dead;
            uint32_t o = 0;
#pragma unroll
            for (int k = 0; k < R; ++k) {
                float q = pad_coordinate<PAD>(pc[k], ext[k], ac);
                int i = (int)rintf(q);
                ok = ok && (uint32_t)i < (uint32_t)ext[k];
                o += (uint32_t)i * stride[k];
            }
            off[0] = ok ? o : GS_OOB;
            w[0] = 1.0f;
        } else if constexpr (MODE == MODE_LINEAR) {
            uint32_t ao[R][2];
            bool av[R][2];
            float aw[R][2];
#pragma unroll
            for (int k = 0; k < R; ++k) {
                float q = pad_coordinate<PAD>(pc[k], ext[k], ac);
                float fl = floorf(q);
                int i0 = (int)fl;
                float t = q - fl;
                aw[k][0] = 1.0f - t;
                aw[k][1] = t;
                av[k][0] = (uint32_t)i0 < (uint32_t)ext[k];
                av[k][1] = (uint32_t)(i0 + 1) < (uint32_t)ext[k];
                ao[k][0] = (uint32_t)i0 * stride[k];
                ao[k][1] = (uint32_t)(i0 + 1) * stride[k];
            }
            // tap index bits: bit k selects the upper tap of axis k
#pragma unroll
            for (int tap = 0; tap < (1 << R); ++tap) {
                bool ok = !dead;
                uint32_t o = 0;
                float ww = 1.0f;
#pragma unroll
                for (int k = R - 1; k >= 0; --k) {
                    int s = (tap >> k) & 1;
                    ok = ok && av[k][s];
                    o += ao[k][s];
                    ww = ww * aw[k][s];
                }
                off[tap] = ok ? o : GS_OOB;
                w[tap] = ww;
            }
        } else {
            uint32_t ao[R][4];
            bool av[R][4];
            float aw[R][4];
#pragma unroll
            for (int k = 0; k < R; ++k) {
                float fl = floorf(pc[k]);
                int i0 = (int)fl;
                float t = pc[k] - fl;
                cubic_weights(t, aw[k]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    int i = i0 - 1 + j;
                    if constexpr (PAD == PAD_ZEROS) {
                        av[k][j] = (uint32_t)i < (uint32_t)ext[k];
                    } else {
                        i = pad_tap<PAD>(i, ext[k], ac);
                        av[k][j] = true;
                    }
                    ao[k][j] = (uint32_t)i * stride[k];
                }
            }
            if constexpr (R == 2) {
#pragma unroll
                for (int jy = 0; jy < 4; ++jy)
#pragma unroll
                    for (int jx = 0; jx < 4; ++jx) {
                        bool ok = !dead && av[1][jy] && av[0][jx];
                        off[jy * 4 + jx] = ok ? ao[1][jy] + ao[0][jx] : GS_OOB;
                        w[jy * 4 + jx] = aw[1][jy] * aw[0][jx];
                    }
            } else {
                // rows (z, y) carry the validity of both; a dead location
                // marks every row out of range; column offsets saturate.
#pragma unroll
                for (int jz = 0; jz < 4; ++jz)
#pragma unroll
                    for (int jy = 0; jy < 4; ++jy) {
                        bool ok = !dead && av[2][jz] && av[1][jy];
                        off[jz * 4 + jy] = ok ? ao[2][jz] + ao[1][jy] : GS_OOB;
                    }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    xoff[j] = av[0][j] ? ao[0][j] : GS_OOB;
                    wz[j] = aw[2][j];
                    wyx[j] = aw[1][j];
                    wx[j] = aw[0][j];
                }
            }
        }
    }
};

// ----------------------------------------------------------- channel loop

template <int R, int MODE, int PAD, typename T, int U>
__device__ __forceinline__ void sample_group(const Taps<R, MODE, PAD, T> &tp, const char *xc,
                                             uint32_t iplane, char *yc, uint32_t oplane,
                                             uint32_t yoff) {
    constexpr int TAPS = Shape<R, MODE>::taps;
    if constexpr (MODE == MODE_NEAREST) {
        typename T::raw_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = T::load_raw(make_rsrc(xc + (size_t)u * iplane, iplane), tp.off[0]);
#pragma unroll
        for (int u = 0; u < U; ++u) T::store_raw(v[u], make_rsrc(yc + (size_t)u * oplane, oplane), yoff);
    } else if constexpr (MODE == MODE_CUBIC && R == 3) {
        // one channel per group: 64 taps, separable x -> y -> z
#pragma unroll
        for (int u = 0; u < U; ++u) {
            rsrc_t xr = make_rsrc(xc + (size_t)u * iplane, iplane);
            float acc = 0.0f;
#pragma unroll
            for (int jz = 0; jz < 4; ++jz) {
                float sz = 0.0f;
#pragma unroll
                for (int jy = 0; jy < 4; ++jy) {
                    float v[4];
#pragma unroll
                    for (int jx = 0; jx < 4; ++jx)
                        v[jx] = T::load(xr, __builtin_elementwise_add_sat(tp.off[jz * 4 + jy], tp.xoff[jx]));
                    float sy = tp.wx[0] * v[0];
                    sy = fmaf(tp.wx[1], v[1], sy);
                    sy = fmaf(tp.wx[2], v[2], sy);
                    sy = fmaf(tp.wx[3], v[3], sy);
                    sz = fmaf(tp.wyx[jy], sy, sz);
                }
                acc = fmaf(tp.wz[jz], sz, acc);
            }
            T::store(acc, make_rsrc(yc + (size_t)u * oplane, oplane), yoff);
        }
    } else {
        float v[U][TAPS];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            rsrc_t xr = make_rsrc(xc + (size_t)u * iplane, iplane);
#pragma unroll
            for (int t = 0; t < TAPS; ++t) v[u][t] = T::load(xr, tp.off[t]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float acc = tp.w[0] * v[u][0];
#pragma unroll
            for (int t = 1; t < TAPS; ++t) acc = fmaf(tp.w[t], v[u][t], acc);
            T::store(acc, make_rsrc(yc + (size_t)u * oplane, oplane), yoff);
        }
    }
}

template <int R, int MODE, int PAD, typename T, bool FUSED>
__global__ __launch_bounds__(kBlock) void grid_sample_kernel(SampleParams p) {
    const int lb = xcd_logical_block(p.nblocks);
    if (lb >= p.nblocks) return;
    const int n = lb / p.tiles_per_n;
    const int tile = lb - n * p.tiles_per_n;
    const uint32_t l = (uint32_t)tile * kBlock + threadIdx.x;
    const bool live = l < p.out_count;
    const uint32_t lc = live ? l : p.out_count - 1;
    const int ac = p.align_corners;

    float g[R];
    if constexpr (FUSED) {
        int d, h, w;
        decompose<R>(lc, p.out_w, p.out_h, p.div_w_m, p.div_w_s, p.div_h_m, p.div_h_s, d, h, w);
        affine_vector<R>(p.theta + (size_t)n * R * (R + 1), d, h, w, p.out_d, p.out_h, p.out_w, ac, g);
    } else {
        const float *gp = p.grid + ((size_t)n * p.out_count + lc) * R;
#pragma unroll
        for (int k = 0; k < R; ++k) g[k] = gp[k];
    }

    const int ext[3] = {p.in_w, p.in_h, p.in_d};
    Taps<R, MODE, PAD, T> tp;
    tp.build(g, ext, ac);

    const uint32_t iplane = p.in_plane_bytes;
    const uint32_t oplane = p.out_plane_bytes;
    const char *xc = (const char *)p.X + (size_t)n * p.C * iplane;
    char *yc = (char *)p.Y + (size_t)n * p.C * oplane;
    const uint32_t yoff = live ? l * (uint32_t)T::bytes : GS_OOB;

    constexpr int U = Shape<R, MODE>::group;
    int c = 0;
    for (; c + U <= p.C; c += U) {
        sample_group<R, MODE, PAD, T, U>(tp, xc, iplane, yc, oplane, yoff);
        xc += (size_t)U * iplane;
        yc += (size_t)U * oplane;
    }
    for (; c < p.C; ++c) {
        sample_group<R, MODE, PAD, T, 1>(tp, xc, iplane, yc, oplane, yoff);
        xc += iplane;
        yc += oplane;
    }
}

// --------------------------------------------------------------- dispatch

static dim3 launch_grid(int nblocks) { return dim3(8 * ((nblocks + 7) / 8)); }

template <int R, bool FUSED, int MODE, int PAD, typename T>
static int launch_one(const SampleParams &p, hipStream_t s) {
    hipLaunchKernelGGL((grid_sample_kernel<R, MODE, PAD, T, FUSED>), launch_grid(p.nblocks),
                       dim3(kBlock), 0, s, p);
    return (int)hipGetLastError();
}

template <int R, bool FUSED, int MODE, int PAD>
static int by_dtype(const SampleParams &p, int dtype, hipStream_t s) {
    switch (dtype) {
    case 0: return launch_one<R, FUSED, MODE, PAD, F32>(p, s);
    case 1: return launch_one<R, FUSED, MODE, PAD, F16>(p, s);
    default: return launch_one<R, FUSED, MODE, PAD, BF16>(p, s);
    }
}

template <int R, bool FUSED, int MODE>
static int by_padding(const SampleParams &p, int padding, int dtype, hipStream_t s) {
    switch (padding) {
    case PAD_ZEROS: return by_dtype<R, FUSED, MODE, PAD_ZEROS>(p, dtype, s);
    case PAD_BORDER: return by_dtype<R, FUSED, MODE, PAD_BORDER>(p, dtype, s);
    default: return by_dtype<R, FUSED, MODE, PAD_REFLECTION>(p, dtype, s);
    }
}

template <int R, bool FUSED>
static int by_mode(const SampleParams &p, int mode, int padding, int dtype, hipStream_t s) {
    switch (mode) {
    case MODE_LINEAR: return by_padding<R, FUSED, MODE_LINEAR>(p, padding, dtype, s);
    case MODE_NEAREST: return by_padding<R, FUSED, MODE_NEAREST>(p, padding, dtype, s);
    default: return by_padding<R, FUSED, MODE_CUBIC>(p, padding, dtype, s);
    }
}

int launch_grid_sample(const SampleParams &p, int rank, bool fused, int mode, int padding,
                       int dtype, hipStream_t stream) {
    if (rank == 2)
        return fused ? by_mode<2, true>(p, mode, padding, dtype, stream)
                     : by_mode<2, false>(p, mode, padding, dtype, stream);
    return fused ? by_mode<3, true>(p, mode, padding, dtype, stream)
                 : by_mode<3, false>(p, mode, padding, dtype, stream);
}

int launch_affine_grid(const AffineParams &p, int rank, hipStream_t stream) {
    if (rank == 2)
        hipLaunchKernelGGL(affine_grid_kernel<2>, launch_grid(p.nblocks), dim3(kBlock), 0, stream, p);
    else
        hipLaunchKernelGGL(affine_grid_kernel<3>, launch_grid(p.nblocks), dim3(kBlock), 0, stream, p);
    return (int)hipGetLastError();
}

}  // namespace gs
