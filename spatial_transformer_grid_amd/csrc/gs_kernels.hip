// gs_kernels.hip -- grid generator and sampler kernels for gfx950.
//
// Sampler layout: a 256-thread block (4 wave64) owns one output tile of one
// image (tile_shape: 1,024 locations in 2D nearest / linear, 4 consecutive
// per lane; 512 in 3D, 2 per lane; 256 for cubic, 1 per lane).  Each lane
// computes its sampling locations, per-axis taps and weights once.
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

#include <type_traits>

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
// The computation type F is float (fp32, fp16 and bf16 theta) or double.
template <int R, typename F>
__device__ __forceinline__ void affine_vector(const F *th, int d, int h, int w, int out_d,
                                              int out_h, int out_w, int ac, F g[R]) {
    F b[3];
    b[0] = base_position<F>(w, out_w, ac);
    b[1] = base_position<F>(h, out_h, ac);
    b[2] = R == 3 ? base_position<F>(d, out_d, ac) : F(0);
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const F *row = th + k * (R + 1);
        F s = row[0] * b[0];
#pragma unroll
        for (int j = 1; j < R; ++j) {
            F prod = row[j] * b[j];
            s = s + prod;
        }
        s = s + row[R];
        g[k] = s;
    }
}

// Element type TT of theta and the grid (AffineGrid page, Type Constraints):
// float, double, _Float16, or __bf16; half types compute in fp32 and round the
// grid to nearest even once, at the store.
template <typename TT>
struct GridElem {
    typedef float F;
    __device__ static F widen(TT v) { return (F)v; }
    __device__ static TT narrow(F v) { return (TT)v; }
};
template <>
struct GridElem<double> {
    typedef double F;
    __device__ static double widen(double v) { return v; }
    __device__ static double narrow(double v) { return v; }
};

// A block writes kAffineLocs consecutive locations of one sample: lane t the
// locations t, t + 256, ... (each store instruction of a wave stays
// contiguous), theta read once.
template <int R, typename TT>
__global__ __launch_bounds__(kBlock) void affine_grid_kernel(AffineParams p) {
    using E = GridElem<TT>;
    using F = typename E::F;
    const int lb = xcd_logical_block(p.nblocks);
    if (lb >= p.nblocks) return;
    const int n = lb / p.tiles_per_n;
    const int tile = lb - n * p.tiles_per_n;
    const TT *tp = (const TT *)p.theta + (size_t)n * R * (R + 1);
    F th[R * (R + 1)];
#pragma unroll
    for (int i = 0; i < R * (R + 1); ++i) th[i] = E::widen(tp[i]);
    TT *gn = (TT *)p.grid + (size_t)n * p.out_count * R;
#pragma unroll
    for (int j = 0; j < kAffineLocs / kBlock; ++j) {
        const uint32_t l = (uint32_t)tile * kAffineLocs + (uint32_t)(j * kBlock) + threadIdx.x;
        if (l < p.out_count) {
            int d, h, w;
            decompose<R>(l, p.out_w, p.out_h, p.div_w_m, p.div_w_s, p.div_h_m, p.div_h_s, d, h, w);
            F g[R];
            affine_vector<R, F>(th, d, h, w, p.out_d, p.out_h, p.out_w, p.align_corners, g);
            TT *out = gn + (size_t)l * R;
#pragma unroll
            for (int k = 0; k < R; ++k) out[k] = E::narrow(g[k]);
        }
    }
}

// ------------------------------------------------------------------ taps

// Per-tap offsets of the tap product, from per-axis parts: a part of an
// invalid tap is `bad`, and the sum saturates, so any invalid tap yields an
// offset >= bad.
template <int R, int K>
struct TapOffsets {
    static constexpr int TAPS = R == 2 ? K * K : K * K * K;
    uint32_t part[R][K];
};

// Interpolate one output of one channel from its precomputed taps; `fetch`
// returns the raw element at a tap offset.  3D cubic is summed separably from
// 16 (z, y) row offsets and 4 x offsets.
template <int R, int MODE, typename T, typename Fetch>
__device__ __forceinline__ float interpolate(const uint32_t *off, const float *w,
                                             const int (&row)[16], const int (&col)[4],
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
                    uint32_t o = min((uint32_t)(row[jz * 4 + jy] + col[jx]), cap);
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

template <int R, int MODE, int PAD, typename T, bool FUSED, bool VEC>
__global__ __launch_bounds__(kBlock) void grid_sample_kernel(SampleParams p) {
    using G = Geo<R, MODE>;
    using raw_t = typename T::raw_t;
    constexpr int Q = G::Q;
    constexpr int K = AxisK<MODE>::K;
    constexpr int TAPS = TapOffsets<R, K>::TAPS;
    constexpr bool SEPARABLE = MODE == MODE_CUBIC && R == 3;
    constexpr int NT = SEPARABLE ? 1 : TAPS;  // precomputed tap offsets / weights
    // LDS staging: up to UMAX channel slots of SS elements in BUDGET elements;
    // the last chunk of every slot holds zeros (the target of invalid taps)
    constexpr int BUDGET = G::stage_bytes / T::bytes;
    constexpr int UMAX = 8;
    constexpr int CH = VEC ? 16 / T::bytes : 1;  // elements per staging chunk
    constexpr int EMAX = (BUDGET / CH + kBlock - 1) / kBlock;  // chunks per thread
    typedef typename std::conditional<VEC, u32x4, raw_t>::type chunk_t;
    constexpr int MAXR = 256;  // input rows (z, y) a staged tile may span
    __shared__ __align__(16) raw_t lds[BUDGET];
    __shared__ int red[kBlock / 64][2 * R];
    __shared__ int row_lo[MAXR], row_hi[MAXR], row_xs[MAXR], row_base[MAXR + 1];
    // row of every chunk of the plan (16-byte chunks only; MAXR = 256 fits a byte)
    constexpr int NCHUNK = VEC ? BUDGET / CH : 1;
    __shared__ uint8_t chunk_row[NCHUNK];
    __shared__ int wave_sum[kBlock / 64];

    if (p.gather_verdicts && gather_chosen(p.gather_verdicts)) return;  // the gather path runs
    const int lb = xcd_logical_block_run_of(p.run);
    if (lb >= p.nblocks) return;
    const int tile = lb % p.tiles_per_n;
    const int ncg = lb / p.tiles_per_n;
    const int cg = ncg % p.cgroups;
    const int n = ncg / p.cgroups;
    const int tx = tile % p.tiles_w;
    const int ty = (tile / p.tiles_w) % p.tiles_h;
    const int tz = tile / (p.tiles_w * p.tiles_h);
    const int t = threadIdx.x;
    const int lrl = p.lanes_row_log2, thl = p.tile_h_log2;
    const int ox0 = tx * p.tile_w + (t & ((1 << lrl) - 1)) * Q;
    const int oy = ty * p.tile_h + ((t >> lrl) & ((1 << thl) - 1));
    const int oz = tz * p.tile_d + (t >> (lrl + thl));
    const int ac = p.align_corners;
    const int ext[3] = {p.in_w, p.in_h, p.in_d};

    // ---- per output: location, taps, weights
    bool live[Q];
    uint32_t yoff[Q];
    AxisTaps<K> ax[Q][R];
    float gq[Q][R];
    if constexpr (!FUSED && R == 2 && Q == 4) {
        if (p.vec_grid) {
            // the lane's 4 grid vectors are 32 contiguous, 32-byte aligned bytes
            const int cy = min(oy, p.out_h - 1);
            const int bx = min(ox0, p.out_w - 4);
            const float4 *g4 = reinterpret_cast<const float4 *>(
                p.grid + ((size_t)n * p.out_count + (uint32_t)cy * (uint32_t)p.out_w + bx) * 2);
            const float4 a = g4[0], b = g4[1];
            gq[0][0] = a.x, gq[0][1] = a.y, gq[1][0] = a.z, gq[1][1] = a.w;
            gq[2][0] = b.x, gq[2][1] = b.y, gq[3][0] = b.z, gq[3][1] = b.w;
        } else {
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int cx = min(ox0 + q, p.out_w - 1), cy = min(oy, p.out_h - 1);
                const float *gp =
                    p.grid + ((size_t)n * p.out_count + (uint32_t)cy * (uint32_t)p.out_w + cx) * 2;
                gq[q][0] = gp[0];
                gq[q][1] = gp[1];
            }
        }
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int ox = ox0 + q;
        live[q] = ox < p.out_w && oy < p.out_h && oz < p.out_d;
        const int cx = min(ox, p.out_w - 1), cy = min(oy, p.out_h - 1), cz = min(oz, p.out_d - 1);
        const uint32_t l =
            ((uint32_t)cz * (uint32_t)p.out_h + (uint32_t)cy) * (uint32_t)p.out_w + cx;
        yoff[q] = live[q] ? l * (uint32_t)T::bytes : GS_OOB;
        float g[R];
        if constexpr (FUSED) {
            affine_vector<R>(p.theta + (size_t)n * R * (R + 1), cz, cy, cx, p.out_d, p.out_h,
                             p.out_w, ac, g);
        } else if constexpr (R == 2 && Q == 4) {
            g[0] = gq[q][0];
            g[1] = gq[q][1];
        } else {
            const float *gp = p.grid + ((size_t)n * p.out_count + l) * R;
#pragma unroll
            for (int k = 0; k < R; ++k) g[k] = gp[k];
        }
        bool any = true;
#pragma unroll
        for (int k = 0; k < R; ++k) {
            float u = unnormalize(g[k], ext[k], ac);
            bool fin = __builtin_isfinite(u);
            float pc = fin ? clampf(u, -kCoordLimit, kCoordLimit) : 0.0f;
            axis_taps<MODE, PAD>(pc, ext[k], ac, ax[q][k]);
            bool axis_any = false;
#pragma unroll
            for (int j = 0; j < K; ++j) {
                ax[q][k].ok[j] = ax[q][k].ok[j] && fin;
                axis_any = axis_any || ax[q][k].ok[j];
            }
            any = any && axis_any;
        }
        // a location that is not finite, or has no in-image tap on some axis,
        // reads nothing: every one of its taps becomes invalid
#pragma unroll
        for (int k = 0; k < R; ++k)
#pragma unroll
            for (int j = 0; j < K; ++j) ax[q][k].ok[j] = ax[q][k].ok[j] && any;
    }

    // ---- bounding box of every valid tap of the block
    int mm[2 * R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        int lo = INT_MAX, nhi = INT_MAX;
#pragma unroll
        for (int q = 0; q < Q; ++q)
#pragma unroll
            for (int j = 0; j < K; ++j)
                if (ax[q][k].ok[j]) {
                    lo = min(lo, ax[q][k].idx[j]);
                    nhi = min(nhi, -ax[q][k].idx[j]);
                }
        mm[2 * k] = lo;
        mm[2 * k + 1] = nhi;
    }
    // the row records of the plan below start empty (block_min's barrier
    // orders this before their first update)
    static_assert(MAXR == kBlock, "one plan row per thread");
    row_lo[t] = INT_MAX;
    row_hi[t] = INT_MIN;
    block_min<2 * R>(mm, red);
    int lo[3] = {0, 0, 0}, span[3] = {1, 1, 1};
    const bool tile_any = mm[0] != INT_MAX;
    if (tile_any) {
#pragma unroll
        for (int k = 0; k < R; ++k) {
            lo[k] = mm[2 * k];
            span[k] = -mm[2 * k + 1] - mm[2 * k] + 1;
        }
    }
    // ---- staging plan: every input row (z, y) of the box gets the interval
    // of 16-byte chunks that covers the x taps the block reads in that row;
    // rows are packed one after another in the LDS slot.
    // The y (and z) taps of an output are consecutive rows for nearest,
    // linear and zero-padded cubic; then an output records its x interval
    // once, at its first row inside the box, and a row's interval is the
    // union of what the K rows (per axis) ending at it recorded.  Otherwise
    // (border / reflection cubic) every tap row records it.
    constexpr bool CONSEC = MODE != MODE_CUBIC || PAD == PAD_ZEROS;
    constexpr int KY = CONSEC ? K : 1, KZ = CONSEC && R == 3 ? K : 1;
    const int64_t nrows = (int64_t)span[1] * span[2];
    int total_chunks = INT_MAX;
    if (tile_any && nrows <= MAXR) {
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            int xl = INT_MAX, xh = INT_MIN;
#pragma unroll
            for (int j = 0; j < K; ++j)
                if (ax[q][0].ok[j]) {
                    xl = min(xl, ax[q][0].idx[j]);
                    xh = max(xh, ax[q][0].idx[j]);
                }
            if constexpr (CONSEC) {
                bool oky = false, okz = R == 2;
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    oky = oky || ax[q][1].ok[j];
                    if (R == 3) okz = okz || ax[q][R - 1].ok[j];
                }
                if (xl <= xh && oky && okz) {
                    const int by = max(ax[q][1].idx[0], lo[1]) - lo[1];
                    const int bz = R == 3 ? max(ax[q][R - 1].idx[0], lo[2]) - lo[2] : 0;
                    const int r = bz * span[1] + by;
                    atomicMin(&row_lo[r], xl);
                    atomicMax(&row_hi[r], xh);
                }
            } else {
#pragma unroll
                for (int jz = 0; jz < (R == 3 ? K : 1); ++jz)
#pragma unroll
                    for (int jy = 0; jy < K; ++jy) {
                        const bool ok =
                            xl <= xh && ax[q][1].ok[jy] && (R == 2 || ax[q][R - 1].ok[jz]);
                        if (ok) {
                            const int r = (R == 3 ? (ax[q][R - 1].idx[jz] - lo[2]) * span[1] : 0) +
                                          ax[q][1].idx[jy] - lo[1];
                            atomicMin(&row_lo[r], xl);
                            atomicMax(&row_hi[r], xh);
                        }
                    }
            }
        }
        __syncthreads();
        // row t of the box: its chunk interval (the union over the rows that
        // end at it), a block-wide prefix sum of the chunk counts (per wave,
        // then the totals of the waves before), and its chunks' entries in
        // the chunk -> row table
        int rl = INT_MAX, rh = INT_MIN;
        if (t < nrows) {
            const int ry = t % span[1], rz = t / span[1];
#pragma unroll
            for (int dz = 0; dz < KZ; ++dz)
#pragma unroll
                for (int dy = 0; dy < KY; ++dy)
                    if (dz <= rz && dy <= ry) {
                        const int sr = t - dz * span[1] - dy;
                        rl = min(rl, row_lo[sr]);
                        rh = max(rh, row_hi[sr]);
                    }
        }
        const bool e = rh >= rl;
        const int xs = e ? (rl & ~(CH - 1)) : 0;
        // (capped: a plan beyond the budget is not staged, and the sum of
        // the counts must not overflow)
        const int cnt = e ? min((rh - xs + CH) / CH, BUDGET) : 0;
        const int incl = wave_inclusive_sum(cnt);
        if ((t & 63) == 63) wave_sum[t >> 6] = incl;
        __syncthreads();
        int before = 0;
        total_chunks = 0;
#pragma unroll
        for (int wv = 0; wv < kBlock / 64; ++wv) {
            const int ws = wave_sum[wv];
            before += wv < (t >> 6) ? ws : 0;
            total_chunks += ws;
        }
        total_chunks = __builtin_amdgcn_readfirstlane(total_chunks);
        const int base = before + incl - cnt;
        row_base[t] = base;
        row_xs[t] = xs;
        if (t == kBlock - 1) row_base[MAXR] = base + cnt;
        if constexpr (VEC) {
            if (total_chunks < NCHUNK)
                for (int c = base; c < base + cnt; ++c) chunk_row[c] = (uint8_t)t;
        }
        __syncthreads();
    }
    // slot stride: the plan plus one zero chunk; as many channels per LDS fill
    // as the budget holds (the next fill is in flight while one is read)
    const int SS = total_chunks < BUDGET ? (total_chunks + 1) * CH : INT_MAX;
    const bool staged = SS <= BUDGET;
    int U = 1;
    if (staged) {
        U = min(UMAX, BUDGET / SS);
        U = (int)min<int64_t>(U, (int64_t)0x7fffffff / p.in_plane_bytes);
    }

    // ---- tap weights
    float w[Q][NT];
    float wz[Q][4], wy[Q][4], wx[Q][4];
    auto tap_weights = [&]() {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        if constexpr (SEPARABLE) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                wx[q][j] = ax[q][0].w[j];
                wy[q][j] = ax[q][1].w[j];
                wz[q][j] = ax[q][2].w[j];
            }
            w[q][0] = 0.0f;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) wx[q][j] = wy[q][j] = wz[q][j] = 0.0f;
#pragma unroll
            for (int tap = 0; tap < TAPS; ++tap) {
                float ww = 1.0f;
                int rem = tap;
#pragma unroll
                for (int k = 0; k < R; ++k) {
                    ww = ww * ax[q][k].w[rem % K];
                    rem /= K;
                }
                w[q][tap] = ww;
            }
        }
    }
    };

    // Tap offsets = row part (z, y) + column part (x).  row_part(q, jz, jy)
    // returns the row part of a valid row; an invalid tap gets `cap`.  For 3D
    // cubic the parts are kept apart (summed per channel): an invalid part is
    // -2^30, which makes the sum negative, i.e. >= 2^31 as unsigned.
    constexpr int BADPART = -(1 << 30);
    uint32_t off[Q][NT];
    int row[Q][16], col[Q][4];
    auto build_offsets = [&](auto row_part, int xscale, uint32_t cap) {
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            int rp[R == 3 ? K : 1][K];
            bool rok[R == 3 ? K : 1][K];
#pragma unroll
            for (int jz = 0; jz < (R == 3 ? K : 1); ++jz)
#pragma unroll
                for (int jy = 0; jy < K; ++jy) {
                    rok[jz][jy] = ax[q][1].ok[jy] && (R == 2 || ax[q][R - 1].ok[jz]);
                    rp[jz][jy] = rok[jz][jy] ? row_part(ax[q][R - 1].idx[jz], ax[q][1].idx[jy]) : 0;
                }
            if constexpr (SEPARABLE) {
#pragma unroll
                for (int jz = 0; jz < 4; ++jz)
#pragma unroll
                    for (int jy = 0; jy < 4; ++jy)
                        row[q][jz * 4 + jy] = rok[jz][jy] ? rp[jz][jy] : BADPART;
#pragma unroll
                for (int jx = 0; jx < 4; ++jx)
                    col[q][jx] = ax[q][0].ok[jx] ? ax[q][0].idx[jx] * xscale : BADPART;
                off[q][0] = 0;
            } else {
#pragma unroll
                for (int tap = 0; tap < TAPS; ++tap) {
                    const int jx = tap % K, jy = (tap / K) % K, jz = R == 3 ? tap / (K * K) : 0;
                    const bool ok = ax[q][0].ok[jx] && rok[jz][jy];
                    off[q][tap] = ok ? (uint32_t)(rp[jz][jy] + ax[q][0].idx[jx] * xscale) : cap;
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) row[q][i] = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) col[q][i] = 0;
            }
        }
    };

    const uint32_t ip = p.in_plane_bytes, op = p.out_plane_bytes;
    const int cbeg = cg * p.cpg;
    const int cend = min(p.C, cbeg + p.cpg);
    const char *xn = (const char *)p.X + ((size_t)n * p.C) * ip;
    char *yn = (char *)p.Y + ((size_t)n * p.C) * op;
    const bool vec_out = p.vec_out != 0;

    if (staged) {
        // ------------------------------------------------ staged in LDS
        // LDS element offset of pixel x of row r within a slot:
        // row_base[r] * CH - row_xs[r] + x; invalid taps read the zero chunk.
        // 3D computes them (and the weights) while the first fill loads; 2D
        // before, which keeps fewer registers live across the copy setup.
        constexpr bool LATE = R == 3;
        auto staged_offsets = [&]() {
            build_offsets(
                [&](int iz, int iy) {
                    const int r = (R == 3 ? (iz - lo[2]) * span[1] : 0) + iy - lo[1];
                    return row_base[r] * CH - row_xs[r];
                },
                1, (uint32_t)(SS - 1));
        };
        if constexpr (!LATE) {
            tap_weights();
            staged_offsets();
        }
        // this thread's copy items: item i = t + e * 256 is chunk c of channel
        // slot u, i = u * total_chunks + c; c's row comes from the chunk ->
        // row table (16-byte chunks) or a branch-free binary search over the
        // row bases.  Items past the plan load through the
        // out-of-range offset (zeros) into slot 0's zero chunk, so the copy
        // loop has no branches: a branch would make the compiler wait for
        // every load in flight before the next one.
        const int nitems = U * total_chunks;
        const float inv_tc = 1.0f / (float)total_chunks;
        const float inv_sy = 1.0f / (float)span[1];
        uint32_t goff[EMAX], loff[EMAX];
#pragma unroll
        for (int e = 0; e < EMAX; ++e) {
            const int i = t + e * kBlock;
            const int u = div_small(i, total_chunks, inv_tc);
            const int c = i - u * total_chunks;
            int r = 0;
            if constexpr (VEC) {
                r = chunk_row[c];
            } else {
#pragma unroll
                for (int step = MAXR / 2; step > 0; step >>= 1)
                    if (row_base[r + step] <= c) r += step;
            }
            const int cx = c - row_base[r];
            int z = 0, y = r;
            if (R == 3) {
                z = div_small(r, span[1], inv_sy);
                y = r - z * span[1];
            }
            const bool in_plan = i < nitems;
            goff[e] = in_plan ? (uint32_t)u * p.in_plane_bytes +
                                    (uint32_t)((((lo[2] + z) * p.in_h + lo[1] + y) * p.in_w +
                                                row_xs[r] + cx * CH) *
                                               T::bytes)
                              : GS_OOB;
            loff[e] = (uint32_t)(in_plan ? u * SS + c * CH : SS - CH) * T::bytes;
        }
        // zero chunk at the end of every slot
        if (t < U) {
            if constexpr (VEC) {
                *(chunk_t *)(lds + t * SS + SS - CH) = chunk_t{0u, 0u, 0u, 0u};
            } else {
                lds[t * SS + SS - CH] = 0;
            }
        }

        auto load_chunk = [&](rsrc_t r, uint32_t o) -> chunk_t {
            if constexpr (VEC) return __builtin_amdgcn_raw_buffer_load_b128(r, (int)o, 0, 0);
            else return T::load_raw(r, o);
        };
        // one resource spans the fill's channels; items of channels past the
        // group's end fall outside it and read zeros
        chunk_t pre[EMAX];
        auto prefetch = [&](int c0) {
            const rsrc_t r = make_rsrc(xn + (size_t)c0 * ip, (uint32_t)min(U, cend - c0) * ip);
#pragma unroll
            for (int e = 0; e < EMAX; ++e) pre[e] = load_chunk(r, goff[e]);
        };
        prefetch(cbeg);
        if constexpr (LATE) {
            tap_weights();
            staged_offsets();
        }
        for (int c0 = cbeg; c0 < cend; c0 += U) {
            __syncthreads();  // the previous fill's LDS reads are done
#pragma unroll
            for (int e = 0; e < EMAX; ++e) *(chunk_t *)((char *)lds + loff[e]) = pre[e];
            __syncthreads();  // this fill is in LDS
            if (c0 + U < cend) prefetch(c0 + U);
            const int nv = min(U, cend - c0);
            for (int u = 0; u < nv; ++u) {
                const int c = c0 + u;
                const raw_t *sl = lds + u * SS;
                const rsrc_t yr = make_rsrc(yn + (size_t)c * op, op);
                raw_t v[Q];
                if constexpr (SEPARABLE) {
#pragma unroll
                    for (int q = 0; q < Q; ++q)
                        v[q] = to_raw<T>(interpolate<R, MODE, T>(
                            off[q], w[q], row[q], col[q], wz[q], wy[q], wx[q], (uint32_t)(SS - 1),
                            [&](uint32_t o) { return sl[o]; }));
                } else {
                    // all LDS reads of the channel first, then the arithmetic
                    raw_t tv[Q][TAPS];
#pragma unroll
                    for (int q = 0; q < Q; ++q)
#pragma unroll
                        for (int tap = 0; tap < TAPS; ++tap) tv[q][tap] = sl[off[q][tap]];
#pragma unroll
                    for (int q = 0; q < Q; ++q) {
                        if constexpr (MODE == MODE_NEAREST) {
                            v[q] = tv[q][0];
                        } else {
                            float acc = w[q][0] * T::from_raw(tv[q][0]);
#pragma unroll
                            for (int tap = 1; tap < TAPS; ++tap)
                                acc = fmaf(w[q][tap], T::from_raw(tv[q][tap]), acc);
                            v[q] = to_raw<T>(acc);
                        }
                    }
                }
                store_outputs<T, Q>(v, yr, yoff, vec_out);
            }
        }
    } else {
        // ------------------------------------------------- direct gather
        tap_weights();
        build_offsets(
            [&](int iz, int iy) { return ((R == 3 ? iz * p.in_h : 0) + iy) * p.in_w * T::bytes; },
            T::bytes, GS_OOB);
        // channels whose loads are all issued before any is used (measured on
        // a random flow: 2D cubic 2 channels 25% faster than 1, 4 slower).
        // Linear stays at 1: more would raise the registers of the whole
        // kernel (the staged path's too: 81 -> 118 VGPRs in 2D, one block
        // less per CU, 1.5% slower on stn2d_batch)
        constexpr int UD = SEPARABLE ? 1
                           : (MODE == MODE_NEAREST ? 8 : (MODE == MODE_CUBIC ? 2 : 1));
        int c = cbeg;
        for (; c + UD <= cend; c += UD) {
            if constexpr (SEPARABLE) {
                const rsrc_t r = make_rsrc(xn + (size_t)c * ip, ip);
                raw_t v[Q];
#pragma unroll
                for (int q = 0; q < Q; ++q)
                    v[q] = to_raw<T>(interpolate<R, MODE, T>(
                        off[q], w[q], row[q], col[q], wz[q], wy[q], wx[q], 0xFFFFFFFFu,
                        [&](uint32_t o) { return T::load_raw(r, o); }));
                store_outputs<T, Q>(v, make_rsrc(yn + (size_t)c * op, op), yoff, vec_out);
            } else {
                raw_t g[UD][Q][TAPS];
#pragma unroll
                for (int u = 0; u < UD; ++u) {
                    const rsrc_t r = make_rsrc(xn + (size_t)(c + u) * ip, ip);
#pragma unroll
                    for (int q = 0; q < Q; ++q)
#pragma unroll
                        for (int tap = 0; tap < TAPS; ++tap) g[u][q][tap] = T::load_raw(r, off[q][tap]);
                }
#pragma unroll
                for (int u = 0; u < UD; ++u) {
                    raw_t v[Q];
#pragma unroll
                    for (int q = 0; q < Q; ++q) {
                        if constexpr (MODE == MODE_NEAREST) {
                            v[q] = g[u][q][0];
                        } else {
                            float acc = w[q][0] * T::from_raw(g[u][q][0]);
#pragma unroll
                            for (int tap = 1; tap < TAPS; ++tap)
                                acc = fmaf(w[q][tap], T::from_raw(g[u][q][tap]), acc);
                            v[q] = to_raw<T>(acc);
                        }
                    }
                    store_outputs<T, Q>(v, make_rsrc(yn + (size_t)(c + u) * op, op), yoff, vec_out);
                }
            }
        }
        for (; c < cend; ++c) {
            const rsrc_t r = make_rsrc(xn + (size_t)c * ip, ip);
            raw_t v[Q];
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                if constexpr (MODE == MODE_NEAREST) {
                    v[q] = T::load_raw(r, off[q][0]);
                } else {
                    v[q] = to_raw<T>(interpolate<R, MODE, T>(
                        off[q], w[q], row[q], col[q], wz[q], wy[q], wx[q], 0xFFFFFFFFu,
                        [&](uint32_t o) { return T::load_raw(r, o); }));
                }
            }
            store_outputs<T, Q>(v, make_rsrc(yn + (size_t)c * op, op), yoff, vec_out);
        }
    }
}

// --------------------------------------------------------------- dispatch

static dim3 launch_grid(int nblocks) { return dim3(8 * ((nblocks + 7) / 8)); }
static dim3 launch_grid_runs(int nblocks, int run) {
    return dim3(8 * run * ((nblocks + 8 * run - 1) / (8 * run)));
}

template <int R, bool FUSED, int MODE, int PAD, typename T>
static int launch_one(const SampleParams &p, bool vec, hipStream_t s) {
    if (vec)
        hipLaunchKernelGGL((grid_sample_kernel<R, MODE, PAD, T, FUSED, true>),
                           launch_grid_runs(p.nblocks, p.run), dim3(kBlock), 0, s, p);
    else
        hipLaunchKernelGGL((grid_sample_kernel<R, MODE, PAD, T, FUSED, false>),
                           launch_grid_runs(p.nblocks, p.run), dim3(kBlock), 0, s, p);
    return (int)hipGetLastError();
}

template <int R, bool FUSED, int MODE, int PAD>
static int by_dtype(const SampleParams &p, int dtype, bool vec, hipStream_t s) {
    switch (dtype) {
    case 0: return launch_one<R, FUSED, MODE, PAD, F32>(p, vec, s);
    case 1: return launch_one<R, FUSED, MODE, PAD, F16>(p, vec, s);
    default: return launch_one<R, FUSED, MODE, PAD, BF16>(p, vec, s);
    }
}

template <int R, bool FUSED, int MODE>
static int by_padding(const SampleParams &p, int padding, int dtype, bool vec, hipStream_t s) {
    switch (padding) {
    case PAD_ZEROS: return by_dtype<R, FUSED, MODE, PAD_ZEROS>(p, dtype, vec, s);
    case PAD_BORDER: return by_dtype<R, FUSED, MODE, PAD_BORDER>(p, dtype, vec, s);
    default: return by_dtype<R, FUSED, MODE, PAD_REFLECTION>(p, dtype, vec, s);
    }
}

template <int R, bool FUSED>
static int by_mode(const SampleParams &p, int mode, int padding, int dtype, bool vec,
                   hipStream_t s) {
    switch (mode) {
    case MODE_LINEAR: return by_padding<R, FUSED, MODE_LINEAR>(p, padding, dtype, vec, s);
    case MODE_NEAREST: return by_padding<R, FUSED, MODE_NEAREST>(p, padding, dtype, vec, s);
    default: return by_padding<R, FUSED, MODE_CUBIC>(p, padding, dtype, vec, s);
    }
}

int launch_grid_sample(const SampleParams &p, int rank, bool fused, int mode, int padding,
                       int dtype, bool vec_in, hipStream_t stream) {
    if (rank == 2)
        return fused ? by_mode<2, true>(p, mode, padding, dtype, vec_in, stream)
                     : by_mode<2, false>(p, mode, padding, dtype, vec_in, stream);
    return fused ? by_mode<3, true>(p, mode, padding, dtype, vec_in, stream)
                 : by_mode<3, false>(p, mode, padding, dtype, vec_in, stream);
}

template <typename TT>
static int affine_launch(const AffineParams &p, int rank, hipStream_t stream) {
    if (rank == 2)
        hipLaunchKernelGGL((affine_grid_kernel<2, TT>), launch_grid(p.nblocks), dim3(kBlock), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((affine_grid_kernel<3, TT>), launch_grid(p.nblocks), dim3(kBlock), 0,
                           stream, p);
    return (int)hipGetLastError();
}

int launch_affine_grid(const AffineParams &p, int rank, hipStream_t stream) {
    switch (p.theta_dtype) {
    case 1: return affine_launch<_Float16>(p, rank, stream);
    case 2: return affine_launch<__bf16>(p, rank, stream);
    case 3: return affine_launch<double>(p, rank, stream);
    default: return affine_launch<float>(p, rank, stream);
    }
}

}  // namespace gs
