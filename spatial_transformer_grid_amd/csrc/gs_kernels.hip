// gs_kernels.hip -- grid generator and sampler kernels for gfx950.
//
// Sampler layout: a 256-thread block (4 wave64) owns one output tile of one
// image, 16 x 16 locations in 2D or 8 x 8 x 4 in 3D, one location per lane.
// Each lane computes its sampling location, per-axis taps and weights once.
// The block then reduces the bounding box of all its taps and picks one of two
// channel loops, uniformly for the whole block:
//
//  * staged: when the box fits the LDS slot (the grid is locally smooth, as
//    for an affine transform or a smooth flow), the block copies the box of U
//    channels at a time from HBM into LDS with row-contiguous loads, and every
//    lane gathers its taps from LDS.  A wave's gather then costs LDS bank
//    cycles instead of one L1 tag lookup per 64-byte segment touched, which is
//    what bounds a direct gather of a rotated or scaled tile.  The next chunk's
//    loads are in flight while the current chunk is interpolated.
//  * direct: otherwise (e.g. i.i.d. random locations) each lane gathers its
//    taps straight from HBM through buffer loads, U channels' loads issued
//    before any of their stores.
//
// Operator definitions: AffineGrid page (Summary: theta applied to evenly
// spaced positions over [-1, 1]); GridSample page (Summary; Attributes
// align_corners, mode, padding_mode).  Cubic uses the cubic convolution kernel
// with a = -0.75 (the cubic_coeff_a default of the Resize page).
#include "gs_device.hpp"
#include "gs_launch.hpp"

#include <limits.h>

namespace gs {

// Flat output location -> (d, h, w) for the grid generator.
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

template <int MODE>
struct AxisK {
    static constexpr int K = MODE == MODE_NEAREST ? 1 : (MODE == MODE_LINEAR ? 2 : 4);
};

template <int K>
struct AxisTaps {
    int idx[K];
    bool ok[K];
    float w[K];
};

// Taps of one axis of n pixels for pixel coordinate pc (finite, |pc| <= 2^24).
template <int MODE, int PAD>
__device__ __forceinline__ void axis_taps(float pc, int n, int ac, AxisTaps<AxisK<MODE>::K> &a) {
    if constexpr (MODE == MODE_NEAREST) {
        float q = pad_coordinate<PAD>(pc, n, ac);
        int i = (int)rintf(q);
        a.idx[0] = i;
        a.ok[0] = (uint32_t)i < (uint32_t)n;
        a.w[0] = 1.0f;
    } else if constexpr (MODE == MODE_LINEAR) {
        float q = pad_coordinate<PAD>(pc, n, ac);
        float fl = floorf(q);
        int i0 = (int)fl;
        float t = q - fl;
        a.idx[0] = i0;
        a.idx[1] = i0 + 1;
        a.ok[0] = (uint32_t)i0 < (uint32_t)n;
        a.ok[1] = (uint32_t)(i0 + 1) < (uint32_t)n;
        a.w[0] = 1.0f - t;
        a.w[1] = t;
    } else {
        // cubic: the location is not padded; each tap is
        float fl = floorf(pc);
        int i0 = (int)fl;
        cubic_weights(pc - fl, a.w);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int i = i0 - 1 + j;
            if constexpr (PAD == PAD_ZEROS) {
                a.idx[j] = i;
                a.ok[j] = (uint32_t)i < (uint32_t)n;
            } else {
                a.idx[j] = pad_tap<PAD>(i, n, ac);
                a.ok[j] = true;
            }
        }
    }
}

// Per-tap offsets of the tap product, from per-axis parts: a part of an
// invalid tap is `bad`, and the sum saturates, so any invalid tap yields an
// offset >= bad.
template <int R, int K>
struct TapOffsets {
    static constexpr int TAPS = R == 2 ? K * K : K * K * K;
    uint32_t part[R][K];
};

// ------------------------------------------------------- block reduction

template <int NV>
__device__ __forceinline__ void block_min(int (&v)[NV], int (*red)[NV]) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v[i] = min(v[i], __shfl_xor(v[i], off, 64));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
#pragma unroll
        for (int i = 0; i < NV; ++i) red[wave][i] = v[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        int m = red[0][i];
#pragma unroll
        for (int wv = 1; wv < kBlock / 64; ++wv) m = min(m, red[wv][i]);
        v[i] = __builtin_amdgcn_readfirstlane(m);
    }
}

// q = f / d for 0 <= f < 2^16, 1 <= d: fp32 estimate, then one correction.
__device__ __forceinline__ int div_small(int f, int d, float inv_d) {
    int q = (int)((float)f * inv_d);
    int r = f - q * d;
    q += (r < 0) ? -1 : (r >= d ? 1 : 0);
    return q;
}

// ---------------------------------------------------------- staging sizes

// LDS staging: U channels per chunk, CAP elements per channel slot, the last
// element of every slot holds 0 (the target of out-of-image taps).
template <int R, int MODE, typename T>
struct Staging {
    static constexpr int U = R == 2 ? (MODE == MODE_CUBIC ? 4 : 8) : (MODE == MODE_CUBIC ? 2 : 4);
    static constexpr int CAP = 16384 / (U * T::bytes);
    static constexpr int ZERO = CAP - 1;
    static constexpr int EMAX = (CAP + kBlock - 1) / kBlock;
};

// Channels per load group of the direct path.
template <int R, int MODE>
struct DirectGroup {
    static constexpr int U = MODE == MODE_NEAREST ? 8
                             : MODE == MODE_LINEAR ? (R == 2 ? 8 : 4)
                                                   : (R == 2 ? 2 : 1);
};

// Interpolate one channel: taps fetched by `fetch(offset)` (raw element).
template <int R, int MODE, typename T, typename Fetch>
__device__ __forceinline__ float interpolate(const uint32_t *off, const float *w,
                                             const uint32_t (&row)[16], const uint32_t (&col)[4],
                                             const float (&wz)[4], const float (&wy)[4],
                                             const float (&wx)[4], uint32_t cap, Fetch fetch) {
    if constexpr (MODE == MODE_CUBIC && R == 3) {
        float acc = 0.0f;
#pragma unroll
        for (int jz = 0; jz < 4; ++jz) {
            float sz = 0.0f;
#pragma unroll
            for (int jy = 0; jy < 4; ++jy) {
                float sy = 0.0f;
#pragma unroll
                for (int jx = 0; jx < 4; ++jx) {
                    uint32_t o = min(__builtin_elementwise_add_sat(row[jz * 4 + jy], col[jx]), cap);
                    sy = fmaf(wx[jx], T::from_raw(fetch(o)), sy);
                }
                sz = fmaf(wy[jy], sy, sz);
            }
            acc = fmaf(wz[jz], sz, acc);
        }
        return acc;
    } else {
        constexpr int TAPS = TapOffsets<R, AxisK<MODE>::K>::TAPS;
        float acc = w[0] * T::from_raw(fetch(off[0]));
#pragma unroll
        for (int t = 1; t < TAPS; ++t) acc = fmaf(w[t], T::from_raw(fetch(off[t])), acc);
        return acc;
    }
}

// --------------------------------------------------------------- sampler

template <int R, int MODE, int PAD, typename T, bool FUSED>
__global__ __launch_bounds__(kBlock) void grid_sample_kernel(SampleParams p) {
    using TS = TileShape<R>;
    using ST = Staging<R, MODE, T>;
    using raw_t = typename T::raw_t;
    constexpr int K = AxisK<MODE>::K;
    constexpr int TAPS = TapOffsets<R, K>::TAPS;
    constexpr bool SEPARABLE = MODE == MODE_CUBIC && R == 3;
    constexpr int NT = SEPARABLE ? 1 : TAPS;  // precomputed tap offsets / weights
    __shared__ raw_t lds[ST::U * ST::CAP];
    __shared__ int red[kBlock / 64][2 * R];

    const int lb = xcd_logical_block(p.nblocks);
    if (lb >= p.nblocks) return;
    const int n = lb / p.tiles_per_n;
    int tile = lb - n * p.tiles_per_n;
    const int tx = tile % p.tiles_w;
    tile /= p.tiles_w;
    const int ty = tile % p.tiles_h;
    const int tz = tile / p.tiles_h;
    const int t = threadIdx.x;
    const int ox = tx * TS::w + t % TS::w;
    const int oy = ty * TS::h + (t / TS::w) % TS::h;
    const int oz = tz * TS::d + t / (TS::w * TS::h);
    const bool live = ox < p.out_w && oy < p.out_h && oz < p.out_d;
    const int cx = min(ox, p.out_w - 1), cy = min(oy, p.out_h - 1), cz = min(oz, p.out_d - 1);
    const uint32_t l = ((uint32_t)cz * (uint32_t)p.out_h + (uint32_t)cy) * (uint32_t)p.out_w + cx;
    const int ac = p.align_corners;

    float g[R];
    if constexpr (FUSED) {
        affine_vector<R>(p.theta + (size_t)n * R * (R + 1), cz, cy, cx, p.out_d, p.out_h, p.out_w,
                         ac, g);
    } else {
        const float *gp = p.grid + ((size_t)n * p.out_count + l) * R;
#pragma unroll
        for (int k = 0; k < R; ++k) g[k] = gp[k];
    }

    // per-axis taps; component k addresses axis k of (W, H, D)
    const int ext[3] = {p.in_w, p.in_h, p.in_d};
    AxisTaps<K> ax[R];
    bool any = true;
#pragma unroll
    for (int k = 0; k < R; ++k) {
        float q = unnormalize(g[k], ext[k], ac);
        bool fin = __builtin_isfinite(q);
        float pc = fin ? clampf(q, -kCoordLimit, kCoordLimit) : 0.0f;
        axis_taps<MODE, PAD>(pc, ext[k], ac, ax[k]);
        bool axis_any = false;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            ax[k].ok[j] = ax[k].ok[j] && fin;
            axis_any = axis_any || ax[k].ok[j];
        }
        any = any && axis_any;
    }
    // a non-finite location, or one with no in-image tap on some axis, reads
    // nothing: clear every axis so all its taps are invalid
#pragma unroll
    for (int k = 0; k < R; ++k)
#pragma unroll
        for (int j = 0; j < K; ++j) ax[k].ok[j] = ax[k].ok[j] && any;

    // bounding box of every valid tap of the block
    int mm[2 * R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        int lo = INT_MAX, nhi = INT_MAX;
#pragma unroll
        for (int j = 0; j < K; ++j)
            if (ax[k].ok[j]) {
                lo = min(lo, ax[k].idx[j]);
                nhi = min(nhi, -ax[k].idx[j]);
            }
        mm[2 * k] = lo;
        mm[2 * k + 1] = nhi;
    }
    block_min<2 * R>(mm, red);
    int lo[3] = {0, 0, 0}, span[3] = {1, 1, 1};
    int area = 0;
    if (mm[0] != INT_MAX) {
        area = 1;
#pragma unroll
        for (int k = 0; k < R; ++k) {
            lo[k] = mm[2 * k];
            span[k] = -mm[2 * k + 1] - mm[2 * k] + 1;
            area *= span[k];
        }
    }

    const uint32_t ip = p.in_plane_bytes, op = p.out_plane_bytes;
    const char *xn = (const char *)p.X + (size_t)n * p.C * ip;
    char *yn = (char *)p.Y + (size_t)n * p.C * op;
    const uint32_t yoff = live ? l * (uint32_t)T::bytes : GS_OOB;
    const int C = p.C;

    // tap weights (products over axes) and, for 3D cubic, per-axis weights
    float w[NT];
    float wz[4] = {0, 0, 0, 0}, wy[4] = {0, 0, 0, 0}, wx[4] = {0, 0, 0, 0};
    if constexpr (SEPARABLE) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            wx[j] = ax[0].w[j];
            wy[j] = ax[1].w[j];
            wz[j] = ax[2].w[j];
        }
        w[0] = 0.0f;
    } else {
#pragma unroll
        for (int tap = 0; tap < TAPS; ++tap) {
            float ww = 1.0f;
            int rem = tap;
#pragma unroll
            for (int k = 0; k < R; ++k) {
                ww = ww * ax[k].w[rem % K];
                rem /= K;
            }
            w[tap] = ww;
        }
    }

    // tap offsets from per-axis parts (stride[k] per unit of axis k)
    auto build_offsets = [&](const uint32_t (&stride)[3], uint32_t bad, uint32_t cap,
                             uint32_t (&off)[NT], uint32_t (&row)[16], uint32_t (&col)[4]) {
        uint32_t part[R][K];
#pragma unroll
        for (int k = 0; k < R; ++k)
#pragma unroll
            for (int j = 0; j < K; ++j)
                part[k][j] = ax[k].ok[j] ? (uint32_t)(ax[k].idx[j] - lo[k]) * stride[k] : bad;
        if constexpr (SEPARABLE) {
#pragma unroll
            for (int jz = 0; jz < 4; ++jz)
#pragma unroll
                for (int jy = 0; jy < 4; ++jy)
                    row[jz * 4 + jy] = __builtin_elementwise_add_sat(part[2][jz], part[1][jy]);
#pragma unroll
            for (int jx = 0; jx < 4; ++jx) col[jx] = part[0][jx];
            off[0] = 0;
        } else {
#pragma unroll
            for (int tap = 0; tap < TAPS; ++tap) {
                uint32_t o = 0;
                int rem = tap;
#pragma unroll
                for (int k = 0; k < R; ++k) {
                    o = __builtin_elementwise_add_sat(o, part[k][rem % K]);
                    rem /= K;
                }
                off[tap] = min(o, cap);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) row[i] = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) col[i] = 0;
        }
    };

    uint32_t off[NT], row[16], col[4];

    if (area <= ST::CAP - 1) {
        // ------------------------------------------------ staged in LDS
        constexpr int U = ST::U, CAP = ST::CAP, ZERO = ST::ZERO, EMAX = ST::EMAX;
        {
            const uint32_t stride[3] = {1u, (uint32_t)span[0], (uint32_t)(span[0] * span[1])};
            build_offsets(stride, 0x40000000u, (uint32_t)ZERO, off, row, col);
        }
        // this thread's share of the box: element f = t + e * 256.  Elements
        // past the box load through the out-of-range offset (value 0) into the
        // zero slot, so the staging code has no branches: a branch would make
        // the compiler wait for every load in flight before the next one.
        const float inv_w = 1.0f / (float)span[0];
        const float inv_wh = 1.0f / (float)(span[0] * span[1]);
        uint32_t goff[EMAX], loff[EMAX];
#pragma unroll
        for (int e = 0; e < EMAX; ++e) {
            const int f = t + e * kBlock;
            int z = 0, rem = f;
            if (R == 3) {
                z = div_small(f, span[0] * span[1], inv_wh);
                rem = f - z * span[0] * span[1];
            }
            const int y = div_small(rem, span[0], inv_w);
            const int x = rem - y * span[0];
            const bool in_box = f < area;
            goff[e] = in_box ? (uint32_t)((((lo[2] + z) * p.in_h + lo[1] + y) * p.in_w + lo[0] + x) *
                                          T::bytes)
                             : GS_OOB;
            loff[e] = in_box ? (uint32_t)f : (uint32_t)ZERO;
        }
        if (t < U) lds[t * CAP + ZERO] = 0;

        raw_t pre[U][EMAX];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool has = u < C;
            const rsrc_t r = make_rsrc(xn + (size_t)(has ? u : 0) * ip, ip);
#pragma unroll
            for (int e = 0; e < EMAX; ++e) pre[u][e] = T::load_raw(r, has ? goff[e] : GS_OOB);
        }
        for (int c0 = 0; c0 < C; c0 += U) {
            __syncthreads();  // the previous chunk's LDS reads are done
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < EMAX; ++e) lds[u * CAP + loff[e]] = pre[u][e];
            __syncthreads();  // this chunk is in LDS
            if (c0 + U < C) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = c0 + U + u;
                    const bool has = c < C;
                    const rsrc_t r = make_rsrc(xn + (size_t)(has ? c : 0) * ip, ip);
#pragma unroll
                    for (int e = 0; e < EMAX; ++e) pre[u][e] = T::load_raw(r, has ? goff[e] : GS_OOB);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u;
                const bool has = c < C;
                const raw_t *s = lds + u * CAP;
                const rsrc_t yr = make_rsrc(yn + (size_t)(has ? c : 0) * op, op);
                const uint32_t yo = has ? yoff : GS_OOB;
                if constexpr (MODE == MODE_NEAREST) {
                    T::store_raw(s[off[0]], yr, yo);
                } else {
                    float v = interpolate<R, MODE, T>(off, w, row, col, wz, wy, wx, (uint32_t)ZERO,
                                                      [&](uint32_t o) { return s[o]; });
                    T::store(v, yr, yo);
                }
            }
        }
    } else {
        // ------------------------------------------------- direct gather
        {
            lo[0] = lo[1] = lo[2] = 0;
            const uint32_t stride[3] = {(uint32_t)T::bytes, (uint32_t)(p.in_w * T::bytes),
                                        (uint32_t)(p.in_w * p.in_h * T::bytes)};
            build_offsets(stride, GS_OOB, 0xFFFFFFFFu, off, row, col);
        }
        constexpr int U = DirectGroup<R, MODE>::U;
        int c = 0;
        for (; c + U <= C; c += U) {
            if constexpr (MODE == MODE_NEAREST) {
                raw_t v[U];
#pragma unroll
                for (int u = 0; u < U; ++u)
                    v[u] = T::load_raw(make_rsrc(xn + (size_t)(c + u) * ip, ip), off[0]);
#pragma unroll
                for (int u = 0; u < U; ++u)
                    T::store_raw(v[u], make_rsrc(yn + (size_t)(c + u) * op, op), yoff);
            } else if constexpr (SEPARABLE) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const rsrc_t r = make_rsrc(xn + (size_t)(c + u) * ip, ip);
                    float v = interpolate<R, MODE, T>(
                        off, w, row, col, wz, wy, wx, 0xFFFFFFFFu,
                        [&](uint32_t o) { return T::load_raw(r, o); });
                    T::store(v, make_rsrc(yn + (size_t)(c + u) * op, op), yoff);
                }
            } else {
                raw_t v[U][TAPS];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const rsrc_t r = make_rsrc(xn + (size_t)(c + u) * ip, ip);
#pragma unroll
                    for (int tap = 0; tap < TAPS; ++tap) v[u][tap] = T::load_raw(r, off[tap]);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float acc = w[0] * T::from_raw(v[u][0]);
#pragma unroll
                    for (int tap = 1; tap < TAPS; ++tap)
                        acc = fmaf(w[tap], T::from_raw(v[u][tap]), acc);
                    T::store(acc, make_rsrc(yn + (size_t)(c + u) * op, op), yoff);
                }
            }
        }
        for (; c < C; ++c) {
            const rsrc_t r = make_rsrc(xn + (size_t)c * ip, ip);
            const rsrc_t yr = make_rsrc(yn + (size_t)c * op, op);
            if constexpr (MODE == MODE_NEAREST) {
                T::store_raw(T::load_raw(r, off[0]), yr, yoff);
            } else {
                float v = interpolate<R, MODE, T>(off, w, row, col, wz, wy, wx, 0xFFFFFFFFu,
                                                  [&](uint32_t o) { return T::load_raw(r, o); });
                T::store(v, yr, yoff);
            }
        }
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
