// gs_resize.hip -- Resize (version 18) kernel for gfx950.
//
// Resize is the axis-aligned special case of the sampler: the sampling
// location of an output element is a per-axis function of its index (Resize
// page, Attributes: coordinate_transformation_mode), so the taps of an output
// row and of an output column are computed once per block axis by axis, and
// the interpolation is separable (linear and cubic are applied axis by axis,
// Attributes: mode).  Up to three trailing axes are resized; the leading axes
// are planes processed one after another.
//
// Layout: a 256-thread block owns one tile of one output depth slice, tile_w x
// tile_h locations with Q consecutive outputs per lane along W.  The input
// rows and columns the tile reads form a rectangle (the locations are
// monotonic along each axis); when that rectangle fits the LDS budget the
// block copies it for U planes at a time with 16-byte loads (the next fill in
// flight while the current one is read) and every lane gathers from LDS,
// otherwise (strong downsampling) lanes gather straight from the input.
// Taps beyond the tensor are clamped to the edge element; with
// exclude_outside their weight is 0 and the others are renormalised
// (Attributes: exclude_outside).
#include "gs_device.hpp"
#include "gs_launch.hpp"

#include <limits.h>

#include <type_traits>

namespace gs {

enum : int { RZ_NEAREST = 0, RZ_LINEAR = 1, RZ_CUBIC = 2 };

template <int MODE>
struct RzK {
    static constexpr int K = MODE == RZ_NEAREST ? 1 : (MODE == RZ_LINEAR ? 2 : 4);
};

// Location x_original of output index x along one axis (Resize page,
// Attributes: coordinate_transformation_mode): half_pixel, pytorch_half_pixel,
// align_corners, asymmetric.  fp32, one rounded operation at a time in the
// order the formulas are written.
__device__ __forceinline__ float resize_location(int x, const ResizeAxis &a, int ct) {
    const float xf = (float)x;
    switch (ct) {
    case 0: return (xf + 0.5f) / a.scale - 0.5f;
    case 1: return a.lr > 1.0f ? (xf + 0.5f) / a.scale - 0.5f : 0.0f;
    case 2: return a.lr > 1.0f ? xf * (float)(a.n - 1) / (a.lr - 1.0f) : 0.0f;
    default: return xf / a.scale;
    }
}

// Keys' cubic convolution kernel (coefficient a) at the distances of the four
// taps floor(p) - 1 .. floor(p) + 2 from p, fractional part t.
__device__ __forceinline__ void keys_weights(float t, float a, float w[4]) {
    const float x0 = t + 1.0f, x1 = t, x2 = 1.0f - t, x3 = 2.0f - t;
    w[0] = fmaf(fmaf(fmaf(a, x0, -5.0f * a), x0, 8.0f * a), x0, -4.0f * a);
    w[1] = fmaf(fmaf(a + 2.0f, x1, -(a + 3.0f)), x1 * x1, 1.0f);
    w[2] = fmaf(fmaf(a + 2.0f, x2, -(a + 3.0f)), x2 * x2, 1.0f);
    w[3] = fmaf(fmaf(fmaf(a, x3, -5.0f * a), x3, 8.0f * a), x3, -4.0f * a);
}

template <int K>
struct RzTaps {
    int idx[K];
    float w[K];
};

// Taps of location p over n input elements (mode, nearest_mode,
// cubic_coeff_a, exclude_outside); indices are clamped into [0, n-1].
template <int MODE>
__device__ __forceinline__ void resize_taps(float p, int n, int nearest_mode, float a, int excl,
                                            RzTaps<RzK<MODE>::K> &t) {
    constexpr int K = RzK<MODE>::K;
    p = clampf(p, -kCoordLimit, kCoordLimit);
    if constexpr (MODE == RZ_NEAREST) {
        float q;
        switch (nearest_mode) {
        case 0: q = ceilf(p - 0.5f); break;   // round_prefer_floor: halfway goes down
        case 1: q = floorf(p + 0.5f); break;  // round_prefer_ceil: halfway goes up
        case 2: q = floorf(p); break;
        default: q = ceilf(p); break;
        }
        t.idx[0] = min(max((int)q, 0), n - 1);
        t.w[0] = 1.0f;
    } else {
        const float fl = floorf(p);
        const float f = p - fl;  // exact
        const int first = (int)fl - (MODE == RZ_CUBIC ? 1 : 0);
        if constexpr (MODE == RZ_LINEAR) {
            t.w[0] = 1.0f - f;
            t.w[1] = f;
        } else {
            keys_weights(f, a, t.w);
        }
        float kept = 0.0f;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int i = first + j;
            if (excl && (i < 0 || i >= n)) t.w[j] = 0.0f;
            kept += t.w[j];
            t.idx[j] = min(max(i, 0), n - 1);
        }
        if (excl) {
#pragma unroll
            for (int j = 0; j < K; ++j) t.w[j] = kept != 0.0f ? t.w[j] / kept : 0.0f;
        }
    }
}

// Sum of one output from its KD x K x K raw taps, x innermost.
template <int MODE, int KD, typename T>
__device__ __forceinline__ float resize_sum(const typename T::raw_t (&v)[KD][RzK<MODE>::K][RzK<MODE>::K],
                                            const float (&wz)[KD], const float (&wy)[RzK<MODE>::K],
                                            const float (&wx)[RzK<MODE>::K]) {
    constexpr int K = RzK<MODE>::K;
    float acc = 0.0f;
#pragma unroll
    for (int z = 0; z < KD; ++z) {
        float sz = 0.0f;
#pragma unroll
        for (int y = 0; y < K; ++y) {
            float sy = wx[0] * T::from_raw(v[z][y][0]);
#pragma unroll
            for (int x = 1; x < K; ++x) sy = fmaf(wx[x], T::from_raw(v[z][y][x]), sy);
            sz = y == 0 ? wy[0] * sy : fmaf(wy[y], sy, sz);
        }
        acc = z == 0 ? wz[0] * sz : fmaf(wz[z], sz, acc);
    }
    return acc;
}

template <int MODE, typename T, bool VEC, bool D3>
__global__ __launch_bounds__(kBlock) void resize_kernel(ResizeParams p) {
    using raw_t = typename T::raw_t;
    constexpr int K = RzK<MODE>::K;
    constexpr int KD = D3 ? K : 1;
    constexpr int Q = RzGeo<MODE, D3>::Q;
    constexpr int CH = VEC ? 16 / T::bytes : 1;
    constexpr int BUDGET = RzGeo<MODE, D3>::stage_bytes / T::bytes;  // elements
    constexpr int EMAX = (BUDGET / CH + kBlock - 1) / kBlock;       // copy items per thread
    constexpr int UMAX = 8;
    typedef typename std::conditional<VEC, u32x4, raw_t>::type chunk_t;
    // the chunk after the budget receives the copy items past the plan
    __shared__ __align__(16) raw_t lds[BUDGET + CH];
    __shared__ int red[kBlock / 64][4];
    // 2D cubic filters in two passes: the staged rows along x for the tile's
    // columns (fp32, HROWS values), then each output along y
    constexpr bool SEP = MODE == RZ_CUBIC && !D3;
    constexpr int HROWS = 3072;
    __shared__ float hbuf[SEP ? HROWS : 1];

    const int lb = xcd_logical_block_runs(p.nblocks);
    if (lb >= p.nblocks) return;
    const int tile = lb % p.tiles_per_plane;
    const int pg = lb / p.tiles_per_plane;
    // With D resized, the output depth slice varies fastest: a run of blocks
    // on one XCD then holds consecutive slices of one tile column, which read
    // the same input slices, and the runs of the neighbouring columns come
    // to the same XCD a round later, so the halo rows and slices are shared
    // in its L2 rather than fetched again by another XCD.
    int tx, ty, od;
    if constexpr (D3) {
        od = tile % p.ax[2].m;
        const int col = tile / p.ax[2].m;
        tx = col % p.tiles_w;
        ty = col / p.tiles_w;
    } else {
        tx = tile % p.tiles_w;
        ty = (tile / p.tiles_w) % p.tiles_h;
        od = tile / (p.tiles_w * p.tiles_h);
    }
    const int t = threadIdx.x;
    const int lrl = p.lanes_row_log2;
    const int ox0 = tx * p.tile_w + (t & ((1 << lrl) - 1)) * Q;
    const int oy = ty * p.tile_h + (t >> lrl);
    const ResizeAxis &aw = p.ax[0], &ah = p.ax[1], &ad = p.ax[2];

    // ---- per-axis taps: Q columns, one row, one depth slice per lane
    RzTaps<K> cx[Q], ry;
    RzTaps<KD == 1 ? 1 : K> dz;
    bool live[Q];
    uint32_t yoff[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int ox = ox0 + q;
        live[q] = ox < aw.m && oy < ah.m;
        resize_taps<MODE>(resize_location(min(ox, aw.m - 1), aw, p.ct), aw.n, p.nearest_mode,
                          p.cubic_a, p.exclude_outside, cx[q]);
        yoff[q] = live[q] ? ((uint32_t)(od * ah.m + oy) * (uint32_t)aw.m + (uint32_t)ox) * T::bytes
                          : GS_OOB;
    }
    resize_taps<MODE>(resize_location(min(oy, ah.m - 1), ah, p.ct), ah.n, p.nearest_mode,
                      p.cubic_a, p.exclude_outside, ry);
    if constexpr (D3) {
        resize_taps<MODE>(resize_location(od, ad, p.ct), ad.n, p.nearest_mode, p.cubic_a,
                          p.exclude_outside, dz);
    } else {
        dz.idx[0] = od < ad.n ? od : 0;
        dz.w[0] = 1.0f;
    }
    float wz[KD], wy[K], wx[Q][K];
#pragma unroll
    for (int j = 0; j < KD; ++j) wz[j] = dz.w[j];
#pragma unroll
    for (int j = 0; j < K; ++j) wy[j] = ry.w[j];
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int j = 0; j < K; ++j) wx[q][j] = cx[q].w[j];

    // ---- input rectangle of the block: columns, rows, depth slices
    int mm[4] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX};
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int j = 0; j < K; ++j) {
            mm[0] = min(mm[0], cx[q].idx[j]);
            mm[1] = min(mm[1], -cx[q].idx[j]);
        }
#pragma unroll
    for (int j = 0; j < K; ++j) {
        mm[2] = min(mm[2], ry.idx[j]);
        mm[3] = min(mm[3], -ry.idx[j]);
    }
    block_min<4>(mm, red);
    int z_lo = dz.idx[0], z_hi = dz.idx[0];
#pragma unroll
    for (int j = 1; j < KD; ++j) {
        z_lo = min(z_lo, dz.idx[j]);
        z_hi = max(z_hi, dz.idx[j]);
    }
    const int xs = mm[0] & ~(CH - 1);
    const int nch = (-mm[1] - xs) / CH + 1;
    const int r_lo = mm[2], nr = -mm[3] - mm[2] + 1, nz = z_hi - z_lo + 1;
    const int64_t plan = (int64_t)nz * nr * nch;  // chunks per plane
    const bool staged = plan * CH <= BUDGET;

    const uint32_t ip = p.in_plane_bytes, op = p.out_plane_bytes;
    const int pbeg = pg * p.ppg;
    const int pend = min(p.P, pbeg + p.ppg);
    const char *xb = (const char *)p.X;
    char *yb = (char *)p.Y;
    const bool vec_out = p.vec_out != 0;

    if (staged) {
        const int SS = (int)plan * CH;  // elements per plane slot
        const int rowlen = nch * CH;
        int U = min(UMAX, BUDGET / SS);
        U = (int)min<int64_t>(U, (int64_t)0x7fffffff / ip);
        // two passes when a plane's filtered rows fit (tile_w is a power of
        // two; at most 256 so that thread t keeps column t % tile_w)
        const int tw = p.tile_w;
        const bool sep = SEP && tw <= kBlock && nr * tw <= HROWS;
        if (sep) U = min(U, HROWS / (nr * tw));
        // pass 1: thread t filters column t % tw of rows t / tw, + 256 / tw, ...
        const int hx = t & (tw - 1), hg = t / tw, hstep = kBlock / tw;
        int hcol[K];
        float hw[K];
        if (sep) {
            RzTaps<K> hc;
            resize_taps<MODE>(resize_location(min(tx * tw + hx, aw.m - 1), aw, p.ct), aw.n,
                              p.nearest_mode, p.cubic_a, p.exclude_outside, hc);
#pragma unroll
            for (int j = 0; j < K; ++j) {
                hcol[j] = hc.idx[j] - xs;
                hw[j] = hc.w[j];
            }
        }
        // LDS element offsets of the taps within a slot
        int colpart[Q][K], rowpart[KD][K];
#pragma unroll
        for (int q = 0; q < Q; ++q)
#pragma unroll
            for (int j = 0; j < K; ++j) colpart[q][j] = cx[q].idx[j] - xs;
#pragma unroll
        for (int z = 0; z < KD; ++z)
#pragma unroll
            for (int j = 0; j < K; ++j)
                rowpart[z][j] = ((dz.idx[z] - z_lo) * nr + ry.idx[j] - r_lo) * rowlen;
        // copy item i = t + e * 256 is chunk c of plane slot u; items past the
        // plan read the out-of-range offset (zeros) into the spare chunk, so
        // the copy has no branch (a branch would serialise the loads)
        const int per = (int)plan;
        const int nitems = U * per;
        const float inv_per = 1.0f / (float)per, inv_nch = 1.0f / (float)nch,
                    inv_nr = 1.0f / (float)nr;
        uint32_t goff[EMAX], loff[EMAX];
#pragma unroll
        for (int e = 0; e < EMAX; ++e) {
            const int i = t + e * kBlock;
            const int u = div_small(i, per, inv_per);
            const int c = i - u * per;
            const int row = div_small(c, nch, inv_nch);
            const int k = c - row * nch;
            const int z = D3 ? div_small(row, nr, inv_nr) : 0;
            const int y = row - z * nr;
            const bool in_plan = i < nitems;
            goff[e] = in_plan ? (uint32_t)u * ip +
                                    (uint32_t)((((z_lo + z) * ah.n + r_lo + y) * aw.n + xs + k * CH) *
                                               T::bytes)
                              : GS_OOB;
            loff[e] = (uint32_t)(in_plan ? u * SS + c * CH : BUDGET) * T::bytes;
        }
        auto load_chunk = [&](rsrc_t r, uint32_t o) -> chunk_t {
            if constexpr (VEC) return __builtin_amdgcn_raw_buffer_load_b128(r, (int)o, 0, 0);
            else return T::load_raw(r, o);
        };
        chunk_t pre[EMAX];
        auto prefetch = [&](int c0) {
            // one resource spans the fill's planes; items of planes past the
            // group's end fall outside it and read zeros
            const rsrc_t r = make_rsrc(xb + (size_t)c0 * ip, (uint32_t)min(U, pend - c0) * ip);
#pragma unroll
            for (int e = 0; e < EMAX; ++e) pre[e] = load_chunk(r, goff[e]);
        };
        prefetch(pbeg);
        for (int c0 = pbeg; c0 < pend; c0 += U) {
            __syncthreads();  // the previous fill's LDS reads are done
#pragma unroll
            for (int e = 0; e < EMAX; ++e) *(chunk_t *)((char *)lds + loff[e]) = pre[e];
            __syncthreads();  // this fill is in LDS
            if (c0 + U < pend) prefetch(c0 + U);
            const int nv = min(U, pend - c0);
            if constexpr (SEP) {
                if (sep) {
                    // the same fp32 operations in the same order as resize_sum:
                    // x first (pass 1), then y (pass 2)
                    for (int u = 0; u < nv; ++u)
                        for (int r = hg; r < nr; r += hstep) {
                            const raw_t *row = lds + u * SS + r * rowlen;
                            float sy = hw[0] * T::from_raw(row[hcol[0]]);
#pragma unroll
                            for (int j = 1; j < K; ++j) sy = fmaf(hw[j], T::from_raw(row[hcol[j]]), sy);
                            hbuf[(u * nr + r) * tw + hx] = sy;
                        }
                    __syncthreads();  // every filtered row is in LDS
                    const int lx = ox0 - tx * tw;
                    for (int u = 0; u < nv; ++u) {
                        const float *hu = hbuf + u * nr * tw;
                        raw_t v[Q];
#pragma unroll
                        for (int q = 0; q < Q; ++q) {
                            float sz = wy[0] * hu[(ry.idx[0] - r_lo) * tw + lx + q];
#pragma unroll
                            for (int j = 1; j < K; ++j)
                                sz = fmaf(wy[j], hu[(ry.idx[j] - r_lo) * tw + lx + q], sz);
                            v[q] = to_raw<T>(wz[0] * sz);
                        }
                        store_outputs<T, Q>(v, make_rsrc(yb + (size_t)(c0 + u) * op, op), yoff, vec_out);
                    }
                    continue;
                }
            }
            // Nearest and linear: each tap's LDS byte address in slot 0, moved
            // on by one slot per plane (one add per tap and plane; indexing
            // from the slot base cost two, the LDS base being added again at
            // every read).  Cubic keeps the row and column parts (64 taps).
            constexpr bool PTR = MODE != RZ_CUBIC;
            typedef __attribute__((address_space(3))) const raw_t *lds_ptr;
            uint32_t tp[PTR ? Q : 1][PTR ? KD : 1][PTR ? K : 1][PTR ? K : 1];
            if constexpr (PTR) {
#pragma unroll
                for (int q = 0; q < Q; ++q)
#pragma unroll
                    for (int z = 0; z < KD; ++z)
#pragma unroll
                        for (int y = 0; y < K; ++y)
#pragma unroll
                            for (int x = 0; x < K; ++x)
                                tp[q][z][y][x] =
                                    (uint32_t)(size_t)((lds_ptr)lds + rowpart[z][y] + colpart[q][x]);
            }
            const uint32_t slot_bytes = (uint32_t)SS * (uint32_t)sizeof(raw_t);
            for (int u = 0; u < nv; ++u) {
                raw_t tv[Q][KD][K][K];
                if constexpr (PTR) {
#pragma unroll
                for (int q = 0; q < Q; ++q)
#pragma unroll
                    for (int z = 0; z < KD; ++z)
#pragma unroll
                        for (int y = 0; y < K; ++y)
#pragma unroll
                            for (int x = 0; x < K; ++x) {
                                tv[q][z][y][x] = *(lds_ptr)(size_t)tp[q][z][y][x];
                                tp[q][z][y][x] += slot_bytes;
                                // opaque to the compiler, which would otherwise
                                // rewrite the address as base + plane offset
                                asm volatile("" : "+v"(tp[q][z][y][x]));
                            }
                } else {
                const raw_t *sl = lds + u * SS;
#pragma unroll
                for (int q = 0; q < Q; ++q)
#pragma unroll
                    for (int z = 0; z < KD; ++z)
#pragma unroll
                        for (int y = 0; y < K; ++y)
#pragma unroll
                            for (int x = 0; x < K; ++x)
                                tv[q][z][y][x] = sl[rowpart[z][y] + colpart[q][x]];
                }
                raw_t v[Q];
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    if constexpr (MODE == RZ_NEAREST) v[q] = tv[q][0][0][0];
                    else v[q] = to_raw<T>(resize_sum<MODE, KD, T>(tv[q], wz, wy, wx[q]));
                }
                store_outputs<T, Q>(v, make_rsrc(yb + (size_t)(c0 + u) * op, op), yoff, vec_out);
            }
        }
    } else {
        // ------------------------------------------------- direct gather
        uint32_t colpart[Q][K], rowpart[KD][K];
#pragma unroll
        for (int q = 0; q < Q; ++q)
#pragma unroll
            for (int j = 0; j < K; ++j) colpart[q][j] = (uint32_t)cx[q].idx[j] * T::bytes;
#pragma unroll
        for (int z = 0; z < KD; ++z)
#pragma unroll
            for (int j = 0; j < K; ++j)
                rowpart[z][j] =
                    ((uint32_t)dz.idx[z] * (uint32_t)ah.n + (uint32_t)ry.idx[j]) * (uint32_t)aw.n *
                    T::bytes;
        for (int c = pbeg; c < pend; ++c) {
            const rsrc_t r = make_rsrc(xb + (size_t)c * ip, ip);
            raw_t tv[Q][KD][K][K];
#pragma unroll
            for (int q = 0; q < Q; ++q)
#pragma unroll
                for (int z = 0; z < KD; ++z)
#pragma unroll
                    for (int y = 0; y < K; ++y)
#pragma unroll
                        for (int x = 0; x < K; ++x)
                            tv[q][z][y][x] = T::load_raw(r, rowpart[z][y] + colpart[q][x]);
            raw_t v[Q];
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                if constexpr (MODE == RZ_NEAREST) v[q] = tv[q][0][0][0];
                else v[q] = to_raw<T>(resize_sum<MODE, KD, T>(tv[q], wz, wy, wx[q]));
            }
            store_outputs<T, Q>(v, make_rsrc(yb + (size_t)c * op, op), yoff, vec_out);
        }
    }
}

// --------------------------------------------------------------- dispatch

template <int MODE, typename T, bool D3>
static int rz_launch(const ResizeParams &p, bool vec, hipStream_t s) {
    const dim3 grid(8 * kRun * ((p.nblocks + 8 * kRun - 1) / (8 * kRun)));
    if (vec)
        hipLaunchKernelGGL((resize_kernel<MODE, T, true, D3>), grid, dim3(kBlock), 0, s, p);
    else
        hipLaunchKernelGGL((resize_kernel<MODE, T, false, D3>), grid, dim3(kBlock), 0, s, p);
    return (int)hipGetLastError();
}

template <int MODE, bool D3>
static int rz_by_dtype(const ResizeParams &p, int dtype, bool vec, hipStream_t s) {
    switch (dtype) {
    case 0: return rz_launch<MODE, F32, D3>(p, vec, s);
    case 1: return rz_launch<MODE, F16, D3>(p, vec, s);
    default: return rz_launch<MODE, BF16, D3>(p, vec, s);
    }
}

template <bool D3>
static int rz_by_mode(const ResizeParams &p, int mode, int dtype, bool vec, hipStream_t s) {
    switch (mode) {
    case RZ_NEAREST: return rz_by_dtype<RZ_NEAREST, D3>(p, dtype, vec, s);
    case RZ_LINEAR: return rz_by_dtype<RZ_LINEAR, D3>(p, dtype, vec, s);
    default: return rz_by_dtype<RZ_CUBIC, D3>(p, dtype, vec, s);
    }
}

int launch_resize(const ResizeParams &p, bool d3, int mode, int dtype, bool vec_in,
                  hipStream_t stream) {
    return d3 ? rz_by_mode<true>(p, mode, dtype, vec_in, stream)
              : rz_by_mode<false>(p, mode, dtype, vec_in, stream);
}

}  // namespace gs
